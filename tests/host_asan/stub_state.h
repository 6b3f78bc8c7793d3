// What the host stand-ins (hip_stub.cpp) saw; read by abi_driver.cpp.
#pragma once

#include "gdn_internal.h"

struct StubState {
  int launches = 0, copies = 0, syncs = 0;
  bool fail_sync = false, fail_launch = false;
  int first = 0, last = 0;
  gdn::PrefillArgs prefill{};
  gdn::DecodeArgs decode{};
};

extern StubState g_stub;
