// internal.h — host-side helpers shared by the C ABI translation units.
#pragma once

#include <string>

namespace pa {

// Records a detail message for pa_last_error() on this thread and returns
// `status`, so call sites can write `return fail(PA_ERR_..., "...")`.
int fail(int status, const std::string& message);
void clear_error();

}  // namespace pa
