// Thread-local error text of the C ABI (muon_last_error), shared by the
// source files that implement entry points.
#pragma once
#include <string>

namespace muon {

// Sets the message muon_last_error() returns on this thread and returns code.
int report_error(int code, const std::string& msg);

}  // namespace muon
