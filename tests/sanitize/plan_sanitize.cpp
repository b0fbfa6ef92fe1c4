// Host driver for a sanitizer build of the planner and argument validator
// (fa_plan.cpp, pure C++): every plan and error path the C ABI offers, over
// ordinary, boundary and overflowing shapes, plus concurrent calls from
// several threads (the detail message is per thread).  Built and run by
// tests/test_sanitize_host.py with AddressSanitizer + UndefinedBehaviorSanitizer
// and, separately, ThreadSanitizer; exits non-zero on the first wrong
// status, and the sanitizers abort on any memory or UB error.

#include <climits>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "fa_internal.h"

static int g_failures = 0;

static void expect(bool ok, const char* what, long long a, long long b) {
    if (!ok) {
        std::fprintf(stderr, "FAIL %s (%lld, %lld)\n", what, a, b);
        ++g_failures;
    }
}

static void plans() {
    const int heads[][2] = {{1, 1}, {2, 2}, {3, 1}, {6, 3}, {8, 8}, {28, 4}, {32, 8}, {32, 32}, {64, 64}, {128, 1}};
    const int lens[] = {0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 300, 2048, 2659, 4096, 16384, 131072};
    const int hds[] = {64, 128, 256};
    for (auto& h : heads)
        for (int S : lens)
            for (int hd : hds)
                for (int causal = 0; causal < 2; ++causal) {
                    fa_plan p;
                    std::memset(&p, 0xab, sizeof p);
                    int st = fa_prefill_plan(h[0], h[1], S, hd, causal, 0, &p);
                    expect(st == FA_OK, "plan", S, hd);
                    if (st == FA_OK) {
                        expect(p.n_q_tiles == (S + p.q_tile - 1) / p.q_tile, "n_q_tiles", S, p.n_q_tiles);
                        expect(p.kv_splits >= 1 && p.kv_splits <= 8, "splits", S, p.kv_splits);
                        expect(p.n_groups >= (long long)p.n_q_tiles * h[0], "groups", S, p.n_groups);
                        expect((p.kv_splits > 1) == (p.workspace_bytes > 0), "workspace", S, p.workspace_bytes);
                        if (S > 0 && p.kv_splits > 1)
                            expect(p.workspace_bytes == fa::workspace_bytes(
                                                            (long long)p.n_q_tiles * h[0],
                                                            (long long)p.n_q_tiles * h[0] * p.kv_splits,
                                                            (long long)p.n_q_tiles * h[0] * p.kv_splits * p.q_tile * hd),
                                   "workspace bytes", S, p.workspace_bytes);
                    }
                    // chunks of every length up to S at a few lengths
                    for (int q : {0, 1, 16, 100, S / 2, S}) {
                        if (q > S) continue;
                        st = fa_prefill_chunk_plan(h[0], h[1], q, S, hd, causal, 160 * 1024, &p);
                        expect(st == FA_OK, "chunk plan", q, S);
                        st = fa_prefill_chunk_plan(h[0], h[1], q, S, hd, causal, 65536, &p);
                        expect(st == (hd == 64 ? FA_OK : FA_ERR_RESOURCE), "chunk plan 64 KiB LDS", q, hd);
                    }
                }
    fa_plan p;
    // shape errors
    expect(fa_prefill_plan(0, 1, 10, 128, 1, 0, &p) == FA_ERR_SHAPE, "heads 0", 0, 0);
    expect(fa_prefill_plan(4, 0, 10, 128, 1, 0, &p) == FA_ERR_SHAPE, "kv heads 0", 0, 0);
    expect(fa_prefill_plan(-4, 2, 10, 128, 1, 0, &p) == FA_ERR_SHAPE, "heads < 0", 0, 0);
    expect(fa_prefill_plan(6, 4, 10, 128, 1, 0, &p) == FA_ERR_SHAPE, "6 % 4", 0, 0);
    expect(fa_prefill_plan(4, 4, -1, 128, 1, 0, &p) == FA_ERR_SHAPE, "S < 0", 0, 0);
    expect(fa_prefill_plan(4, 4, INT_MIN, 128, 1, 0, &p) == FA_ERR_SHAPE, "S = INT_MIN", 0, 0);
    expect(fa_prefill_chunk_plan(4, 4, 10, 9, 128, 1, 0, &p) == FA_ERR_SHAPE, "kv < q", 0, 0);
    expect(fa_prefill_chunk_plan(4, 4, -3, 9, 128, 1, 0, &p) == FA_ERR_SHAPE, "q < 0", 0, 0);
    for (int hd : {0, -128, 1, 32, 96, 127, 129, 192, 512, INT_MAX})
        expect(fa_prefill_plan(4, 4, 10, hd, 1, 0, &p) == FA_ERR_HEAD_DIM, "head_dim", hd, 0);
    // sizes that overflow the grid, the tensor offsets or the buffer offsets
    expect(fa_prefill_plan(INT_MAX, 1, INT_MAX, 128, 1, 0, &p) == FA_ERR_SHAPE, "huge grid", 0, 0);
    expect(fa_prefill_plan(1 << 20, 1 << 20, 1 << 20, 256, 1, 0, &p) == FA_ERR_SHAPE, "huge kv heads", 0, 0);
    expect(fa_prefill_plan(65536, 1, INT_MAX, 128, 0, 0, &p) == FA_ERR_SHAPE, "huge tensor", 0, 0);
    // LDS limits
    expect(fa_prefill_plan(4, 4, 10, 256, 1, 65536, &p) == FA_ERR_RESOURCE, "lds 256", 0, 0);
    expect(fa_prefill_plan(4, 4, 10, 128, 1, 81920, &p) == FA_OK, "lds 128 fits", 0, 0);
    expect(fa_prefill_plan(4, 4, 10, 128, 1, 81919, &p) == FA_ERR_RESOURCE, "lds 128 one short", 0, 0);
    // NULL plan pointer: validation only
    expect(fa_prefill_plan(32, 32, 2659, 128, 1, 0, nullptr) == FA_OK, "null plan", 0, 0);
    expect(std::strlen(fa_prefill_last_error()) == 0, "no error after success", 0, 0);
    expect(fa_prefill_plan(6, 4, 10, 128, 1, 0, nullptr) == FA_ERR_SHAPE, "null plan error", 0, 0);
    expect(std::strlen(fa_prefill_last_error()) > 0, "detail after error", 0, 0);
}

static void validation() {
    char* base = reinterpret_cast<char*>(0x100000);
    const void *q = base, *k = base + (1 << 24), *v = base + (2 << 24);
    void* out = base + (3 << 24);
    using fa::validate_call;
    expect(validate_call(q, k, v, out, 4, 4, 64, 64, 128, 0.1f, 4) == FA_OK, "valid", 0, 0);
    expect(validate_call(nullptr, k, v, out, 4, 4, 64, 64, 128, 0.1f, 4) == FA_ERR_NULL, "null q", 0, 0);
    expect(validate_call(nullptr, nullptr, nullptr, nullptr, 4, 4, 0, 0, 128, 0.1f, 4) == FA_OK, "empty", 0, 0);
    expect(validate_call(base + 8, k, v, out, 4, 4, 64, 64, 128, 0.1f, 4) == FA_ERR_ALIGN, "align", 0, 0);
    expect(validate_call(q, k, v, out, 4, 4, 64, 64, 128, __builtin_nanf(""), 4) == FA_ERR_SCALE, "nan", 0, 0);
    expect(validate_call(q, k, v, out, 4, 4, 64, 64, 128, __builtin_inff(), 4) == FA_ERR_SCALE, "inf", 0, 0);
    expect(validate_call(q, k, v, base + (1 << 24) + 4096, 4, 4, 64, 64, 128, 0.1f, 4) == FA_ERR_ALIAS, "alias k", 0, 0);
    expect(validate_call(q, k, v, base, 4, 4, 64, 64, 128, 0.1f, 2) == FA_ERR_ALIAS, "alias q", 0, 0);
    // extreme sizes: offsets are formed in 64 bits
    expect(validate_call(q, k, v, out, 1 << 16, 1, INT_MAX, INT_MAX, 256, 0.1f, 4) != FA_OK, "overlap huge", 0, 0);
    for (int dt : {-1, 0, 1, 2, 3, 100})
        for (int ot : {-1, 0, 1, 2, 3}) {
            const bool ok = (dt == FA_DTYPE_F16 || dt == FA_DTYPE_BF16) && (ot == FA_DTYPE_F32 || ot == dt);
            expect((fa::check_dtypes(dt, ot) == FA_OK) == ok, "dtypes", dt, ot);
        }
    for (int s = -5; s < 20; ++s) expect(fa_prefill_strerror(s) != nullptr && fa_prefill_strerror(s)[0], "strerror", s, 0);
}

static void threads() {
    std::vector<std::thread> pool;
    int bad[8] = {0};
    for (int t = 0; t < 8; ++t)
        pool.emplace_back([t, &bad] {
            for (int i = 0; i < 2000; ++i) {
                fa_plan p;
                const int nq = (t % 2) ? 6 : 8;
                const int st = fa_prefill_chunk_plan(nq, 4, 1 + (i % 300), 4096, 128, 1, 0, &p);
                const bool want_err = nq % 4 != 0;
                if ((st != FA_OK) != want_err) ++bad[t];
                const char* msg = fa_prefill_last_error();
                if (want_err != (msg[0] != '\0')) ++bad[t];
            }
        });
    for (auto& th : pool) th.join();
    for (int t = 0; t < 8; ++t) expect(bad[t] == 0, "thread", t, bad[t]);
}

int main(int argc, char** argv) {
    const bool only_threads = argc > 1 && std::strcmp(argv[1], "threads") == 0;
    if (!only_threads) {
        plans();
        validation();
    }
    threads();
    if (g_failures) {
        std::fprintf(stderr, "%d failures\n", g_failures);
        return 1;
    }
    std::printf("plan_sanitize: ok\n");
    return 0;
}
