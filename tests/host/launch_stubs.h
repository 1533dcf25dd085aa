// Record of the last stubbed launch (see launch_stubs.cpp).
#pragma once

#include "params.h"
#include "qjl_params.h"

namespace kvq {

struct StubLog {
  int encode_calls = 0, decode_calls = 0, attend_calls = 0, qjl_calls = 0, scratch_lookups = 0;
  int d = 0, bits = 0, stages = 0, nqw = 0, m = 0;
  EncodeArgs enc{};
  DecodeArgs dec{};
  AttendArgs att{};
  QjlArgs qjl{};
};

extern StubLog g_stub;

}  // namespace kvq
