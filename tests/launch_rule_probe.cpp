// Host-only probe of the launch rules in dispatch_common.hpp (built and run by
// tests/test_launch_rules.py on the CPU): for n = 1..32, the dynamic LDS that
// lets n workgroups of a launch share a CU, and the read-ahead size rule.
#include <cstdio>

#include "dispatch_common.hpp"

int main() {
    for (int n = 1; n <= 32; ++n)
        std::printf("lds %d %d\n", n, moe_dispatch::lds_for_workgroups_per_cu(n));
    std::printf("per_cu %d\n", moe_dispatch::kLdsPerCu);
    const long long mb = 1ll << 20;
    std::printf("fits %d %d %d\n", (int)moe_dispatch::read_ahead_fits(160 * mb, 0),
                (int)moe_dispatch::read_ahead_fits(160 * mb - 64, 16), (int)moe_dispatch::read_ahead_fits(160 * mb, 1));
    return 0;
}
