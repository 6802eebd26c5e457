// What the host-memory HIP test double records (see hip_host_double.cpp).
#pragma once

namespace dbl {
struct HostDouble {
    long long launches = 0, bad_launches = 0, copies = 0, records = 0, waits = 0, state_writes = 0;
    long long last_grid = 0, last_block = 0;
    int live_events = 0, last_wait_count = 0;
    int last_int[3] = {0, 0, 0};
    void* last_ptr = nullptr;
    bool capturing = false;
};
extern HostDouble g;
}  // namespace dbl
