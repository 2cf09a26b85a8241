// Host-side checks of liblores's C ABI (csrc/lores_api.cpp) built with
// AddressSanitizer and UndefinedBehaviorSanitizer against launch_stubs.cpp:
// layout planning, validation, launch grouping, the windowed states' step
// bookkeeping and the precision assignment, with no GPU.  Prints "host check
// ok" and exits 0 on success; a failed check prints its line and exits 1.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "../../include/lores.h"
#include "../../quantized_linear_recurrence_amd/csrc/lores_internal.h"
#include "launch_log.h"

static int g_fail = 0;
#define CHECK(c)                                                                        \
    do {                                                                                \
        if (!(c)) {                                                                     \
            std::printf("FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #c,               \
                        lores_last_error());                                            \
            ++g_fail;                                                                   \
        }                                                                               \
    } while (0)

struct Buf {
    void *p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes) : n((bytes + 255) / 256 * 256) { p = std::aligned_alloc(256, n); }
    ~Buf() { std::free(p); }
};

static size_t size_of(int B, int H, int dk, int dv, const std::vector<uint8_t> &prec, int axis = 0,
                      int window = 1) {
    size_t n = 0;
    int rc = window > 1 || axis ? lores_state_alloc_window(B, H, dk, dv, prec.data(), axis, window,
                                                           nullptr, &n, nullptr, nullptr)
                                : lores_state_alloc(B, H, dk, dv, prec.data(), nullptr, &n,
                                                    nullptr, nullptr);
    return rc == LORES_OK ? n : 0;
}

// device-like argument block: every pointer 256-byte aligned, large enough
struct Args {
    Buf q{1 << 20}, k{1 << 20}, v{1 << 20}, a{1 << 20}, b{1 << 20}, o{1 << 20};
};

static int step(lores_state *st, Args &x, uint64_t t, int per_channel = 0, int delta = 1) {
    return lores_decode_step(st, x.q.p, x.k.p, x.v.p, 0, (const float *)x.a.p, per_channel,
                             (const float *)x.b.p, delta, 7, t, 0, 0, (float *)x.o.p, nullptr);
}

int main() {
    // hand-computed sizes: codes d_v_pad * chunk bytes, scales d_v_pad * 4,
    // window (W - 1)(d_v_pad + d_k + 1) * 4 padded to 16, each segment 256-aligned
    CHECK(size_of(1, 1, 64, 64, {LORES_INT8}) == 4096 + 256);
    CHECK(size_of(1, 1, 64, 64, {LORES_INT4}) == 2048 + 256);
    CHECK(size_of(1, 1, 64, 64, {LORES_FP32}) == 16384);
    CHECK(size_of(1, 1, 64, 64, {LORES_INT8}, LORES_SCALE_KEY) == 4096 + 256);
    CHECK(size_of(1, 1, 128, 64, {LORES_INT8}, LORES_SCALE_KEY) == 8192 + 512);
    CHECK(size_of(1, 1, 64, 64, {LORES_INT8}, 0, 3) == 4096 + 256 + 1536);   // 2*(64+2*64)*4 = 1536
    CHECK(size_of(1, 1, 64, 1, {LORES_INT6}) == 48 * 64 + 256);             // 3 chunks of 16 B per row
    // d_k > 128: two half rows, each whole chunks (int4 at 160: 2 x 48 B, int6 at 224: 2 x 96 B)
    CHECK(size_of(1, 1, 160, 64, {LORES_INT4}) == 96 * 64 + 256);
    CHECK(size_of(1, 1, 224, 64, {LORES_INT6}) == 192 * 64 + 256);
    CHECK(size_of(1, 1, 256, 64, {LORES_INT4}) == 128 * 64 + 256);

    // plans over many shapes: segments in bounds, disjoint, 256-aligned
    const int dks[] = {32, 64, 96, 128, 160, 192, 224, 256};
    const int dvs[] = {1, 64, 65, 128, 150, 200, 256};
    std::vector<std::vector<uint8_t>> mixes = {{2}, {3, 2}, {0, 1, 2, 3, 4, 5}, {5, 5, 4}, {1, 3}};
    for (int dk : dks)
        for (int dv : dvs)
            for (auto &mix : mixes)
                for (int axis = 0; axis < 2; ++axis)
                    for (int W : {1, 4}) {
                        const int B = 3, H = (int)mix.size();
                        size_t n = 0;
                        int rc = lores_state_alloc_window(B, H, dk, dv, mix.data(), axis, W, nullptr,
                                                          &n, nullptr, nullptr);
                        CHECK(rc == LORES_OK);
                        Buf buf(n);
                        lores_state *st = nullptr;
                        g_launches.clear();
                        CHECK(lores_state_alloc_window(B, H, dk, dv, mix.data(), axis, W, buf.p, &n,
                                                       nullptr, &st) == LORES_OK);
                        CHECK(g_launches.v.size() == 1 && g_launches.v[0].kind == "fill_zero");
                        lores_layout lay;
                        CHECK(lores_state_layout(st, &lay) == LORES_OK);
                        CHECK(lay.total_bytes == n && lay.window == W && lay.scale_axis == axis);
                        std::vector<std::pair<int64_t, int64_t>> seg;
                        for (int c = 0; c < LORES_NUM_PREC; ++c) {
                            if (!lay.n_class[c]) continue;
                            seg.push_back({lay.codes_offset[c],
                                           lay.codes_offset[c] + (int64_t)B * lay.n_class[c] *
                                                                     lay.unit_code_bytes[c]});
                            if (lay.scales_offset[c] >= 0)
                                seg.push_back({lay.scales_offset[c],
                                               lay.scales_offset[c] + (int64_t)B * lay.n_class[c] *
                                                                          lay.unit_scales * 4});
                            if (lay.window_offset[c] >= 0)
                                seg.push_back({lay.window_offset[c],
                                               lay.window_offset[c] + (int64_t)B * lay.n_class[c] *
                                                                          lay.unit_window_bytes[c]});
                        }
                        for (size_t i = 0; i < seg.size(); ++i) {
                            CHECK(seg[i].first % 256 == 0 && seg[i].second <= (int64_t)n);
                            for (size_t j = 0; j < seg.size(); ++j)
                                if (i != j)
                                    CHECK(seg[i].second <= seg[j].first || seg[j].second <= seg[i].first);
                        }
                        lores_state_free(st);
                    }

    Args x;
    // d_k = 256: rows split across lane pairs, 32 rows per task; three
    // classes, one launch each
    for (int dv : {1, 32, 33, 100, 256}) {
        const std::vector<uint8_t> prec = {2, 3, 1, 3};
        const int B = 2, H = (int)prec.size();
        size_t n = size_of(B, H, 256, dv, prec);
        Buf buf(n);
        lores_state *st = nullptr;
        CHECK(lores_state_alloc(B, H, 256, dv, prec.data(), buf.p, &n, nullptr, &st) == LORES_OK);
        g_launches.clear();
        CHECK(step(st, x, 1) == LORES_OK);
        CHECK(g_launches.v.size() == 3);
        for (auto &l : g_launches.v) {
            CHECK(l.p1 < 0);
            CHECK(l.n_rb == (dv + 31) / 32);
            CHECK(l.groups[0] == (l.Hc[0] * l.n_rb + lores::kWavesPerGroup - 1) /
                                     lores::kWavesPerGroup);
        }
        lores_state_free(st);
    }
    // work-groups of each step launch cover its tasks: a fused int pair counts
    // only the unpaired rest of either class, in groups of kPairWavesPerGroup
    // wavefronts; other launches count all tasks of a class in groups of
    // kWavesPerGroup
    // (split rows at d_k > 128 as well: 32-row tasks)
    {
        const std::vector<std::vector<uint8_t>> mixes = {
            {2, 3}, {2, 2, 2, 3}, {3, 3, 3, 3, 3, 2}, {3, 4, 4}, {1, 2, 2}, {1, 3, 3, 3},
            {2, 3, 4}, {0, 1, 2, 3, 4, 5}, {2, 2, 2, 2, 2, 2, 2, 2, 2, 3}};
        for (int dk : {128, 160, 256})
        for (auto &prec : mixes)
            for (int dv : {1, 64, 100, 128, 256}) {
                const int B = 2, H = (int)prec.size();
                size_t n = size_of(B, H, dk, dv, prec);
                Buf buf(n);
                lores_state *st = nullptr;
                CHECK(lores_state_alloc(B, H, dk, dv, prec.data(), buf.p, &n, nullptr, &st) ==
                      LORES_OK);
                g_launches.clear();
                CHECK(step(st, x, 1) == LORES_OK);
                int heads = 0;
                for (auto &l : g_launches.v) {
                    const bool pair = l.p1 == LORES_INT4 || l.p1 == LORES_INT6;
                    const bool pair_ints = pair && l.p0 != LORES_BF16;
                    const int n0 = l.Hc[0] * l.n_rb, n1 = l.p1 >= 0 ? l.Hc[1] * l.n_rb : 0;
                    CHECK(l.n_rb == (dk > 128 ? (dv + 31) / 32 : (dv + 63) / 64));
                    heads += l.Hc[0] + (l.p1 >= 0 ? l.Hc[1] : 0);
                    if (pair_ints) {
                        const int paired = n0 < n1 ? n0 : n1, w = lores::kPairWavesPerGroup;
                        CHECK(l.groups[0] == (n0 - paired + w - 1) / w);
                        CHECK(l.groups[1] == (n1 - paired + w - 1) / w);
                    } else {
                        const int w = lores::kWavesPerGroup;
                        CHECK(l.groups[0] == (n0 + w - 1) / w);
                        if (l.p1 >= 0) CHECK(l.groups[1] == (n1 + w - 1) / w);
                    }
                }
                CHECK(heads == H);
                lores_state_free(st);
            }
    }
    // split rows fuse the same pairs
    for (int dk : {160, 192, 224, 256}) {
        const std::vector<std::pair<std::vector<uint8_t>, std::string>> cases = {
            {{2, 3, 2, 3}, "launch_step_int8_int4"}, {{4, 3}, "launch_step_int4_int6"},
            {{1, 2, 2}, "launch_step_bf16_int8"}, {{3, 1}, "launch_step_bf16_int4"}};
        for (auto &c : cases) {
            const int H = (int)c.first.size();
            size_t n = size_of(2, H, dk, 100, c.first);
            Buf buf(n);
            lores_state *st = nullptr;
            CHECK(lores_state_alloc(2, H, dk, 100, c.first.data(), buf.p, &n, nullptr, &st) ==
                  LORES_OK);
            g_launches.clear();
            CHECK(step(st, x, 1) == LORES_OK);
            CHECK(g_launches.v.size() == 1 && g_launches.v[0].kind == c.second);
            int32_t nl = 0;
            CHECK(lores_step_launches(st, &nl) == LORES_OK && nl == 1);
            lores_state_free(st);
        }
    }
    // launch grouping: a fused pair for value rows, one launch per class for key columns
    {
        std::vector<uint8_t> prec = {2, 3, 2, 3};
        size_t n = size_of(4, 4, 128, 128, prec);
        Buf buf(n);
        lores_state *st = nullptr;
        CHECK(lores_state_alloc(4, 4, 128, 128, prec.data(), buf.p, &n, nullptr, &st) == LORES_OK);
        g_launches.clear();
        CHECK(step(st, x, 1) == LORES_OK);
        CHECK(g_launches.v.size() == 1 && g_launches.v[0].kind == "launch_step_int8_int4");
        int32_t nl = 0;
        CHECK(lores_step_launches(st, &nl) == LORES_OK && nl == 1);
        // invalid arguments launch nothing
        g_launches.clear();
        CHECK(step(st, x, 0) == LORES_EINVAL);
        CHECK(step(st, x, 1, 0, 2) == LORES_EINVAL);
        CHECK(lores_decode_step(st, nullptr, x.k.p, x.v.p, 0, (const float *)x.a.p, 0,
                                (const float *)x.b.p, 1, 0, 1, 0, 0, (float *)x.o.p, nullptr) ==
              LORES_EINVAL);
        CHECK(lores_decode_step(st, (char *)x.q.p + 2, x.k.p, x.v.p, 0, (const float *)x.a.p, 0,
                                (const float *)x.b.p, 1, 0, 1, 0, 0, (float *)x.o.p, nullptr) ==
              LORES_EINVAL);
        CHECK(lores_decode_step(st, x.q.p, x.k.p, x.v.p, 0, (const float *)x.a.p, 0,
                                (const float *)x.b.p, 1, 0, 1, -1, 0, (float *)x.o.p, nullptr) ==
              LORES_EINVAL);
        CHECK(lores_state_set_rounding(st, 7) == LORES_EINVAL);
        CHECK(g_launches.v.empty());
        CHECK(std::strlen(lores_last_error()) > 0);
        CHECK(lores_state_set_rounding(st, LORES_ROUND_NEAREST) == LORES_OK);
        CHECK(std::strlen(lores_last_error()) == 0);
        lores_state_free(st);

        n = size_of(4, 4, 128, 128, prec, LORES_SCALE_KEY);
        Buf kb(n);
        CHECK(lores_state_alloc_axis(4, 4, 128, 128, prec.data(), LORES_SCALE_KEY, kb.p, &n, nullptr,
                                     &st) == LORES_OK);
        g_launches.clear();
        CHECK(step(st, x, 1) == LORES_OK);
        CHECK(g_launches.v.size() == 2 && g_launches.v[0].kind == "launch_step_key_int8" &&
              g_launches.v[1].kind == "launch_step_key_int4");
        lores_state_free(st);
        // key columns over three row blocks: one unit per three-wavefront group
        n = size_of(4, 4, 128, 150, prec, LORES_SCALE_KEY);
        Buf k3(n);
        CHECK(lores_state_alloc_axis(4, 4, 128, 150, prec.data(), LORES_SCALE_KEY, k3.p, &n, nullptr,
                                     &st) == LORES_OK);
        g_launches.clear();
        CHECK(step(st, x, 1) == LORES_OK);
        CHECK(g_launches.v.size() == 2);
        for (auto &l : g_launches.v) CHECK(l.n_rb == 3 && l.groups[0] == l.Hc[0]);
        lores_state_free(st);
    }
    // windowed states: positions follow t, steps must come in order
    {
        std::vector<uint8_t> prec = {2, 1, 3};
        const int W = 4;
        size_t n = size_of(2, 3, 64, 64, prec, 0, W);
        Buf buf(n);
        lores_state *st = nullptr;
        CHECK(lores_state_alloc_window(2, 3, 64, 64, prec.data(), 0, W, buf.p, &n, nullptr, &st) ==
              LORES_OK);
        for (uint64_t t = 1; t <= 9; ++t) {
            g_launches.clear();
            CHECK(step(st, x, t) == LORES_OK);
            int windowed = 0;
            for (auto &l : g_launches.v)
                if (l.kind == "window") {
                    ++windowed;
                    CHECK(l.wpos == (int)((t - 1) % W) + 1 && l.window == W);
                } else {
                    CHECK(l.kind == "launch_step_bf16");
                }
            CHECK(windowed == 2);
            lores_layout lay;
            CHECK(lores_state_layout(st, &lay) == LORES_OK && lay.window_fill == (int)(t % W));
        }
        g_launches.clear();
        CHECK(step(st, x, 12) == LORES_EINVAL);              // the buffer holds token 9's window
        CHECK(step(st, x, 10, 1) == LORES_EINVAL);           // the window's tokens are scalar-decay
        CHECK(g_launches.v.empty());
        Buf out(1 << 20);
        g_launches.clear();
        CHECK(lores_dequant_state(st, (float *)out.p, nullptr) == LORES_OK);
        int replays = 0;
        for (auto &l : g_launches.v)
            if (l.kind == "window_dequant") {
                ++replays;
                CHECK(l.wpos == 1);
            }
        CHECK(replays == 2);
        CHECK(lores_quant_state(st, (const float *)out.p, 0, 0, 0, nullptr) == LORES_OK);
        lores_layout lay;
        CHECK(lores_state_layout(st, &lay) == LORES_OK && lay.window_fill == 0);
        CHECK(step(st, x, 10) == LORES_EINVAL);
        CHECK(step(st, x, 13) == LORES_OK);
        lores_state_free(st);
    }
    // windows whose tokens carry one decay per key channel: one kind of decay
    // per window, passed to the window's launches and to its dequantization
    {
        std::vector<uint8_t> prec = {2, 3};
        const int W = 3;
        size_t n = size_of(2, 2, 64, 64, prec, 0, W);
        Buf buf(n);
        lores_state *st = nullptr;
        CHECK(lores_state_alloc_window(2, 2, 64, 64, prec.data(), 0, W, buf.p, &n, nullptr, &st) ==
              LORES_OK);
        g_launches.clear();
        CHECK(step(st, x, 1, 1) == LORES_OK);
        CHECK(g_launches.v.size() == 2);
        for (auto &l : g_launches.v) CHECK(l.kind == "window_pc" && l.win_pc == 1 && l.wpos == 1);
        g_launches.clear();
        CHECK(step(st, x, 2, 0) == LORES_EINVAL);
        CHECK(g_launches.v.empty());
        Buf out(1 << 20);
        CHECK(lores_dequant_state(st, (float *)out.p, nullptr) == LORES_OK);
        CHECK(g_launches.v.size() == 2);
        for (auto &l : g_launches.v) CHECK(l.kind == "window_dequant" && l.win_pc == 1);
        CHECK(step(st, x, 2, 1) == LORES_OK);
        CHECK(step(st, x, 3, 1) == LORES_OK);
        lores_layout lay;
        CHECK(lores_state_layout(st, &lay) == LORES_OK && lay.window_fill == 0);
        g_launches.clear();
        CHECK(step(st, x, 4, 0) == LORES_OK);              // a new window: a scalar decay again
        for (auto &l : g_launches.v) CHECK(l.kind == "window" && l.win_pc == 0);
        lores_state_free(st);
    }
    // launch errors: an error left on the thread by earlier work is not the
    // call's own; a launch that fails is reported, and a windowed state then
    // keeps its position, so the same step can be issued again
    {
        std::vector<uint8_t> prec = {2, 3};
        const int W = 4;
        size_t n = size_of(2, 2, 64, 64, prec, 0, W);
        Buf buf(n);
        lores_state *st = nullptr;
        lores_layout lay;
        g_sticky_error = hipErrorInvalidValue;
        CHECK(lores_state_alloc_window(2, 2, 64, 64, prec.data(), 0, W, buf.p, &n, nullptr, &st) ==
              LORES_OK);
        g_sticky_error = hipErrorInvalidValue;
        CHECK(step(st, x, 1) == LORES_OK);
        CHECK(lores_state_layout(st, &lay) == LORES_OK && lay.window_fill == 1);
        g_fail_next_launch = true;
        CHECK(step(st, x, 2) == LORES_EHIP);
        CHECK(std::strstr(lores_last_error(), "launch failed") != nullptr);
        CHECK(lores_state_layout(st, &lay) == LORES_OK && lay.window_fill == 1);
        CHECK(step(st, x, 2) == LORES_OK);
        CHECK(lores_state_layout(st, &lay) == LORES_OK && lay.window_fill == 2);
        Buf out(1 << 20);
        g_sticky_error = hipErrorInvalidValue;
        CHECK(lores_dequant_state(st, (float *)out.p, nullptr) == LORES_OK);
        g_sticky_error = hipErrorInvalidValue;
        CHECK(lores_quant_state(st, (const float *)out.p, 0, 0, 0, nullptr) == LORES_OK);
        g_fail_next_launch = true;
        CHECK(lores_dequant_state(st, (float *)out.p, nullptr) == LORES_EHIP);
        g_fail_next_launch = true;
        CHECK(lores_quant_state(st, (const float *)out.p, 0, 0, 0, nullptr) == LORES_EHIP);
        CHECK(g_sticky_error == hipSuccess && !g_fail_next_launch);
        lores_state_free(st);
        std::vector<uint8_t> one = {2};
        n = size_of(1, 1, 64, 64, one);
        Buf b1(n);
        g_fail_next_launch = true;
        CHECK(lores_state_alloc(1, 1, 64, 64, one.data(), b1.p, &n, nullptr, &st) == LORES_EHIP);
    }
    // decay statistic and precision assignment
    {
        const int H = 6;
        std::vector<float> alpha(4 * H);
        for (int i = 0; i < 4 * H; ++i) alpha[i] = 0.5f + 0.08f * (float)(i % H);
        double stat[H];
        CHECK(lores_decay_stat(alpha.data(), 4, H, 1, stat) == LORES_OK);
        for (int h = 1; h < H; ++h) CHECK(stat[h] > stat[h - 1]);
        double frac[2] = {0.5, 0.5};
        uint8_t tiers[2] = {LORES_INT8, LORES_INT4}, out[H];
        CHECK(lores_assign_precision(stat, H, frac, tiers, 2, out) == LORES_OK);
        for (int h = 0; h < H; ++h) CHECK(out[h] == (h >= 3 ? LORES_INT8 : LORES_INT4));
        alpha[3] = 0.0f;
        CHECK(lores_decay_stat(alpha.data(), 4, H, 1, stat) == LORES_EINVAL);
        stat[2] = std::nan("");
        CHECK(lores_assign_precision(stat, H, frac, tiers, 2, out) == LORES_EINVAL);
        tiers[1] = 9;
        stat[2] = 0.0;
        CHECK(lores_assign_precision(stat, H, frac, tiers, 2, out) == LORES_EINVAL);
    }
    if (g_fail) {
        std::printf("%d host checks failed\n", g_fail);
        return 1;
    }
    std::printf("host check ok\n");
    return 0;
}
