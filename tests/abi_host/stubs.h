// Counters of the host-only launcher stand-ins (stubs.cpp).
#pragma once

namespace stub {
extern int launches;
extern int last_T, last_d, last_E, last_k, last_f;
extern int last_kind;
extern int events_recorded;
}  // namespace stub
