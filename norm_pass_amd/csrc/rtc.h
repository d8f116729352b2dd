// Runtime specialisation of elementwise chains with hipRTC (DeepJIT write-up,
// hotelren.com/news/5350627, sections 3.1-3.3 and 6.2-6.4).
#pragma once

#include <string>

#include "internal.h"

namespace np {

// Generate, compile and load a kernel for this op list / dtypes / n (n == 0:
// any n) on the current device; cached for the life of the process.
// Returns NP_OK, NP_ECOMPILE (log holds the compiler output) or NP_ELAUNCH.
int rtc_prepare(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, std::string* log);

// Launch a prepared specialisation if one matches (16-byte aligned buffers
// only). Returns false when none matches; *e holds the launch status otherwise.
bool rtc_launch(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, hipStream_t s,
                hipError_t* e);

// Generated source for a chain (exposed for tests of the generator).
std::string rtc_source(const ChainArgs& a, int n_inputs, int in_dt, int out_dt, int64_t n);

// Unload every cached module (streams that used them must be idle).
void rtc_clear();

}  // namespace np
