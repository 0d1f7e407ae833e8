// Error reporting shared by the host-only entry points: sets the calling
// thread's tdx_last_error() text (cleared on TDX_OK) and returns code.
#ifndef TDX_ERRORS_H
#define TDX_ERRORS_H

namespace tdx {
int report(int code, const char* msg);
}

#endif
