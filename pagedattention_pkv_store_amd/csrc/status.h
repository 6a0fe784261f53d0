// Shared by the host and device translation units of libpkv: the thread-local
// message behind pkv_last_error().
#ifndef PKV_STATUS_H_
#define PKV_STATUS_H_

#include <string>

namespace pkv {

// Record `msg` as this thread's last error and return `code`.
int fail(int code, const std::string& msg);

}  // namespace pkv

#endif  // PKV_STATUS_H_
