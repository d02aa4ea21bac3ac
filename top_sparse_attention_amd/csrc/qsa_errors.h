// Error text shared by the C-ABI layer and the other host code of libqsa.
#pragma once

namespace qsa {

// Sets the calling thread's qsa_last_error() text and returns `status`
// (defined with the C-ABI layer).
int set_error(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace qsa
