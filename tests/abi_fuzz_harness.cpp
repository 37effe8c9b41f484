// Fuzz of the C-ABI validation and launch-planning paths, built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized.py).  No
// GPU use: only the check predicates (which validate and never launch or dereference)
// and the host-only plan diagnostic are called, with random and boundary sizes,
// strides and fake addresses (null, misaligned, at the top of the address space,
// overlapping).  Any sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <random>
#include "adaln.h"
static const int64_t V[] = {0, 1, 2, 7, 8, 9, 16, 63, 64, 127, 128, 1024, 2048, 3072, 4096, 4104, 8192, 8200,
                            65535, 1 << 20, (int64_t)1 << 31, ((int64_t)1 << 31) - 1, ((int64_t)1 << 32) + 8,
                            (int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX, INT64_MAX - 7, -1, -8, INT64_MIN};
int main() {
    std::mt19937_64 rng(1);
    auto pick = [&]() { return V[rng() % (sizeof(V) / sizeof(V[0]))]; };
    auto ptr = [&]() -> const adaln_bf16* {
        const uint64_t k = rng() % 6;
        if (k == 0) return nullptr;
        if (k == 1) return (const adaln_bf16*)(uintptr_t)(0x1000 + 2 * (rng() % 64));
        if (k == 2) return (const adaln_bf16*)(uintptr_t)(UINT64_MAX - 15);
        return (const adaln_bf16*)(uintptr_t)((rng() % (1ull << 44)) & ~15ull);
    };
    long n = 0, ok = 0;
    for (int it = 0; it < 2000000; ++it) {
        const int64_t B = pick(), T = pick(), H = pick(), s0 = pick(), s1 = pick(), s2 = pick();
        const float eps = (rng() % 4 == 0) ? -1.0f : 1e-6f;
        adaln_status st;
        switch (rng() % 8) {
            case 0: st = adaln_check_layernorm_modulate(ptr(), ptr(), ptr(), (adaln_bf16*)ptr(), B, T, H, s0, s1, eps); break;
            case 1: st = adaln_check_rmsnorm_scale_shift(ptr(), ptr(), ptr(), ptr(), (adaln_bf16*)ptr(), B, T, H, s0, s1, eps); break;
            case 2: st = adaln_check_residual_gate_rmsnorm_scale_shift(ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), (adaln_bf16*)ptr(), (adaln_bf16*)ptr(), B, T, H, s0, s1, s2, eps); break;
            case 3: st = adaln_check_residual_gate_layernorm_modulate(ptr(), ptr(), ptr(), ptr(), ptr(), (adaln_bf16*)ptr(), (adaln_bf16*)ptr(), B, T, H, s0, s1, s2, eps); break;
            case 4: st = adaln_check_layernorm_modulate_fp8_quant(ptr(), ptr(), ptr(), (const float*)ptr(), (uint8_t*)ptr(), B, T, H, s0, s1, eps); break;
            case 5: st = adaln_check_qk_rmsnorm_rope(ptr(), ptr(), ptr(), ptr(), (const float*)ptr(), (adaln_bf16*)ptr(), (adaln_bf16*)ptr(), T, B, H, s0, s1, pick(), eps); break;
            case 6: st = adaln_check_residual_gate_channel_first(ptr(), ptr(), ptr(), (adaln_bf16*)ptr(), B, H, T, s0); break;
            default: {
                int64_t out[11];
                const int64_t res[3] = {s0, s1, s2};
                st = adaln_diag_launch_plan((int)(rng() % 7) - 1, B, H, T, res, pick(), out);
                if (st == ADALN_OK) {
                    // a plan has groups, groups per block and rows per block, and its
                    // grid holds fewer than 2^32 work-items
                    if (out[3] < 1 || out[4] < 1 || out[5] < 1 || out[9] < 1 ||
                        out[9] > (int64_t)0xFFFFFFFF / out[10]) {
                        std::printf("bad plan\n");
                        return 1;
                    }
                }
            }
        }
        ++n;
        if (st == ADALN_OK) ++ok;
        (void)adaln_status_string(st);
    }
    // structured phase: distinct regions, realistic and boundary sizes and strides
    const int64_t Hs[] = {8, 16, 520, 1024, 2048, 2056, 3072, 4096, 4104, 8192};
    const int64_t Ts[] = {1, 2, 7, 128, 4096, 4333, 4608, (int64_t)1 << 20, (int64_t)1 << 28, (int64_t)1 << 34};
    const int64_t Bs[] = {0, 1, 2, 3, 64, 1 << 16};
    long acc2 = 0;
    for (int it = 0; it < 2000000; ++it) {
        const int64_t H = Hs[rng() % 10], T = Ts[rng() % 10], B = Bs[rng() % 6];
        const int64_t strides[] = {0, H, H - 8, H + 8, 6 * H, -8, 3 * H, H / 2};
        const int64_t s0 = strides[rng() % 8], s1 = strides[rng() % 8], s2 = strides[rng() % 8];
        auto region = [&](int k) -> uintptr_t {
            // regions 1 TiB apart, some shifted by a few elements so that they overlap
            return ((uintptr_t)(k + 1) << 40) + ((rng() % 8 == 0) ? 16 * (rng() % 4) : 0) -
                   ((rng() % 16 == 0) ? ((uintptr_t)1 << 40) : 0);
        };
        const adaln_bf16 *x = (const adaln_bf16*)region(0), *r = (const adaln_bf16*)region(1),
                         *g = (const adaln_bf16*)region(2), *sc = (const adaln_bf16*)region(3),
                         *sh = (const adaln_bf16*)region(4), *w = (const adaln_bf16*)region(5);
        adaln_bf16 *y = (adaln_bf16*)region(6), *ro = (adaln_bf16*)region(7);
        adaln_status st;
        switch (rng() % 6) {
            case 0: st = adaln_check_layernorm_modulate(x, sc, sh, y, B, T, H, s0, s1, 1e-6f); break;
            case 1: st = adaln_check_rmsnorm_scale_shift(x, w, sc, sh, y, B, T, H, s0, s1, 1e-6f); break;
            case 2: st = adaln_check_residual_gate_rmsnorm_scale_shift(r, x, g, w, sc, sh, ro, y, B, T, H, s0, s1, s2, 1e-6f); break;
            case 3: st = adaln_check_residual_gate_layernorm_modulate(r, x, g, sc, sh, ro, y, B, T, H, s0, s1, s2, 1e-6f); break;
            case 4: st = adaln_check_layernorm_modulate_fp8_quant(x, sc, sh, (const float*)g, (uint8_t*)y, B, T, H, s0, s1, 0.0f); break;
            default: st = adaln_check_residual_gate_channel_first(r, x, g, y, B, T, H, s0); break;
        }
        if (st == ADALN_OK) ++acc2;
        int64_t out[11];
        if (B > 0 && T > 0 && B <= INT64_MAX / T) {
            const int64_t res[3] = {1 + (int64_t)(rng() % 8192), (int64_t)(rng() % 8192),
                                    (int64_t)(rng() % 8192)};
            (void)adaln_diag_launch_plan((int)(rng() % 5), B * T, H, T, res,
                                         (int64_t)(rng() % 512), out);
        }
    }
    std::printf("structured accepted %ld\n", acc2);
    int w, l, c;
    for (int64_t h : V) (void)adaln_reduction_layout(h, &w, &l, &c);
    std::printf("calls %ld, accepted %ld\n", n, ok);
    return 0;
}
