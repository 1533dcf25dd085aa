// Stand-ins for the kernel launchers of libkvq (kernels.hip, attend.hip, qjl.hip) so that
// the host half of the library (argument checks, codebooks, plans: api.cpp, codebooks.cpp)
// can be built and run without a GPU, under AddressSanitizer and UBSan. Each stub keeps a
// copy of the argument block it was given and returns success; nothing is launched.
#include <hip/hip_runtime.h>

#include "launch_stubs.h"

namespace kvq {

StubLog g_stub;

hipError_t launch_encode(const EncodeArgs& a, int d, int bits, int stages, hipStream_t) {
  ++g_stub.encode_calls;
  g_stub.enc = a;
  g_stub.d = d;
  g_stub.bits = bits;
  g_stub.stages = stages;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int d, int bits, int stages, hipStream_t) {
  ++g_stub.decode_calls;
  g_stub.dec = a;
  g_stub.d = d;
  g_stub.bits = bits;
  g_stub.stages = stages;
  return hipSuccess;
}

hipError_t launch_attend(const AttendArgs& a, int d, int bits, int nqw, hipStream_t) {
  ++g_stub.attend_calls;
  g_stub.att = a;
  g_stub.d = d;
  g_stub.bits = bits;
  g_stub.nqw = nqw;
  return hipSuccess;
}

hipError_t launch_qjl(const QjlArgs& a, int d, int m, hipStream_t) {
  ++g_stub.qjl_calls;
  g_stub.qjl = a;
  g_stub.d = d;
  g_stub.m = m;
  return hipSuccess;
}

hipError_t attend_scratch(void** ptr) {
  ++g_stub.scratch_lookups;
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7000000));  // a fake, aligned device address
  return hipSuccess;
}

}  // namespace kvq
