// errors.hpp -- the library's thread-local last-error text, shared by the
// translation units that hold entry points (qrp_last_error() reads it).
#pragma once

#include <stdint.h>

#include <string>

namespace qrp {

// Record `msg` as the calling thread's last error and return `code`.
int32_t set_error(int32_t code, const std::string& msg);
// Forget the calling thread's last error (each entry point starts with it).
void clear_error();

}  // namespace qrp
