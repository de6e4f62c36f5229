// The launch log kept by the test-double launchers (stub_launchers.cpp).
#pragma once
#include "kernels.hpp"

namespace la {

struct StubLog {
  int rope = 0, prefill = 0, merge = 0, decode = 0, combine = 0, backward = 0;
  RopeArgs rope_q{}, rope_k{};
  RopeAngles angles{};
  PrefillArgs pre{}, pre_merge{};
  DecodeArgs dec{};
  CombineArgs comb{};
  BwdArgs bwd{};
  int D = 0, G = 0, dt = -1;
};
extern StubLog g_stub;

}  // namespace la
