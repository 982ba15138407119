// host_checks.cpp -- host-only checks of the library's plan logic and
// workspace record, built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_host_sanitizers.py (plan.cpp is pure host code, so it links
// without the HIP runtime).  Exit status 0 = every check passed; any
// sanitizer report aborts the run.
#include <stdio.h>
#include <stdlib.h>

#include <thread>
#include <vector>

#include "plan.h"

static int g_fail = 0;
#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                       \
        }                                                                   \
    } while (0)

namespace hy {
const char* last_error_text();
}

// Every layout a plan computes stays inside the buffers it sizes.
static void check_layout(const hy::Plan& p)
{
    CHECK(p.workspace_bytes >= p.tw_bytes);
    CHECK(p.tw_bytes >= (size_t)p.tw_elems * 8);
    for (int s = 0; s < p.nseg; ++s) {
        CHECK(p.seg[s].off >= 0);
        CHECK(p.seg[s].off + (int64_t)(p.seg[s].radix - 1) * p.seg[s].ns <= p.tw_elems);
    }
    CHECK(p.inter_copies == 1 || p.inter_copies == 2);
    CHECK(p.inter_offset + p.inter_bytes <= p.workspace_bytes);
    if (p.inter_copies == 2) {
        // the chain's second copy lies after the first and inside the workspace
        CHECK(p.fwd_offset[0] == p.inter_offset);
        CHECK(p.fwd_offset[1] >= p.inter_offset + p.inter_bytes);
        CHECK(p.fwd_offset[1] + (size_t)(p.chunk_pairs * p.fwd_pair_bytes) <= p.fwd2_offset[1]);
        CHECK(p.fwd2_offset[1] + (size_t)(p.chunk_pairs * p.fwd_pair_bytes2) <= p.workspace_bytes);
        CHECK(p.fwd_offset[1] + (size_t)(p.chunk_pairs * p.fwd_pair_bytes) <= p.workspace_bytes);
    }
    CHECK(p.stage_offset + p.stage_bytes <= p.workspace_bytes || p.stage_bytes == 0);
    CHECK(p.spectrum_bytes > 0);
    if (p.path == HYENA_PATH_FOURSTEP1D || p.path == HYENA_PATH_ROWCOL2D) {
        CHECK(p.chunk_pairs >= 1);
        const int64_t per = p.fwd_pair_bytes > p.spec_pair_bytes ? p.fwd_pair_bytes : p.spec_pair_bytes;
        CHECK((size_t)(p.chunk_pairs * per) <= p.inter_bytes);
    }
    if (p.path == HYENA_PATH_ROWCOL3D) CHECK(p.inter2_offset + 1 <= p.inter_offset + p.inter_bytes);
    if (p.path == HYENA_PATH_FOURSTEP1D) CHECK(p.M1 * p.M2 == p.M);
}

static void plans()
{
    const int64_t Ns[] = {4, 5, 7, 8, 100, 256, 1000, 2048, 4096, 8191, 8192, 8193, 65536, 100000,
                          1 << 20, 2097152, 2097153, 0, -3};
    const int32_t dts[] = {HYENA_F32, HYENA_BF16, HYENA_F16, 9};
    int ok = 0, rejected = 0;
    for (int64_t N : Ns)
        for (int32_t io : dts)
            for (int32_t sp : dts)
                for (int32_t order : {0, 1, 2, 8, 9})
                    for (int32_t path : {0, 1, 2, 3, 4, 7})
                        for (int32_t flags : {0, 1, 2}) {
                            hy::Plan p;
                            const int64_t dims[1] = {N};
                            const hyena_status st =
                                hy::plan_build(p, 2, N, 7, order, dims, 1, io, sp, path, flags);
                            if (st == HYENA_OK) {
                                ++ok;
                                check_layout(p);
                            } else {
                                ++rejected;
                                CHECK(hy::last_error_text()[0] != '\0');
                            }
                        }
    const int64_t sides[] = {2, 4, 8, 64, 256, 512, 1024, 2048, 3};
    for (int64_t X : sides)
        for (int64_t Y : sides) {
            hy::Plan p;
            const int64_t dims[2] = {X, Y};
            if (hy::plan_build(p, 1, X * Y, 5, 2, dims, 2, HYENA_F32, HYENA_F32, 0, 0) == HYENA_OK) {
                ++ok;
                check_layout(p);
            } else {
                ++rejected;
            }
            for (int64_t Z : {4, 16, 64}) {
                hy::Plan q;
                const int64_t d3[3] = {X, Y, Z};
                if (hy::plan_build(q, 1, X * Y * Z, 3, 1, d3, 3, HYENA_BF16, HYENA_BF16, 0, 0) ==
                    HYENA_OK) {
                    ++ok;
                    check_layout(q);
                } else {
                    ++rejected;
                }
            }
        }
    // chains that walk several chunks keep two copies of the intermediate
    {
        const int64_t d1[1] = {65536}, d2[2] = {512, 512}, d3[3] = {64, 64, 64};
        hy::Plan a, b, c, e;
        CHECK(hy::plan_build(a, 1, 65536, 768, 2, d1, 1, HYENA_F32, HYENA_F32, 0, 0) == HYENA_OK);
        CHECK(hy::plan_build(b, 3, 512 * 512, 34, 2, d2, 2, HYENA_F32, HYENA_F32, 0, 0) == HYENA_OK);
        CHECK(hy::plan_build(c, 2, 64 * 64 * 64, 32, 2, d3, 3, HYENA_F32, HYENA_F32, 0, 0) ==
              HYENA_OK);
        CHECK(hy::plan_build(e, 1, 65536, 32, 2, d1, 1, HYENA_F32, HYENA_F32, 0, 0) == HYENA_OK);
        for (const hy::Plan* q : {&a, &b, &c}) {
            check_layout(*q);
            CHECK(q->inter_copies == 2);
        }
        check_layout(e);
        CHECK(e.inter_copies == 1);  // 16 pair slots: one chunk
        ok += 4;
    }
    // null dims, bad ndims
    hy::Plan p;
    CHECK(hy::plan_build(p, 1, 8, 1, 1, nullptr, 1, 0, 0, 0, 0) == HYENA_ERR_INVALID_ARGUMENT);
    const int64_t d4[4] = {4, 4, 4, 4};
    CHECK(hy::plan_build(p, 1, 256, 1, 1, d4, 4, 0, 0, 0, 0) == HYENA_ERR_UNSUPPORTED);
    CHECK(ok > 100 && rejected > 100);
    printf("plans: %d built, %d rejected\n", ok, rejected);
}

static void workspace_record()
{
    char buf[4096];
    const uint64_t A = 1001, B = 1002;
    CHECK(!hy::ws_record_use(buf, 256, A));
    hy::ws_record_init(buf, 256, A);
    CHECK(hy::ws_record_use(buf, 256, A));
    CHECK(!hy::ws_record_use(buf, 256, B));
    // released: no longer usable, and a second release is a no-op
    CHECK(hy::ws_record_release(buf, A));
    CHECK(!hy::ws_record_release(buf, A));
    CHECK(!hy::ws_record_use(buf, 256, A));
    // another plan initialising the same bytes takes them over
    hy::ws_record_init(buf, 256, A);
    hy::ws_record_init(buf, 256, B);
    CHECK(!hy::ws_record_use(buf, 256, A));
    CHECK(hy::ws_record_use(buf, 256, B));
    // a workspace that overlaps from below or above drops the older record
    hy::ws_record_init(buf + 512, 256, A);
    CHECK(hy::ws_record_use(buf + 512, 256, A));
    hy::ws_record_init(buf + 256, 512, B);  // [256, 768) overlaps [512, 768)
    CHECK(!hy::ws_record_use(buf + 512, 256, A));
    hy::ws_record_init(buf + 2048, 256, A);
    hy::ws_record_init(buf + 1024, 4096 - 1024, B);  // reaches over buf + 2048
    CHECK(!hy::ws_record_use(buf + 2048, 256, A));
    // adjacent, non-overlapping records coexist
    hy::ws_record_drop(A);
    hy::ws_record_drop(B);
    CHECK(hy::ws_record_count() == 0);
    hy::ws_record_init(buf, 1024, A);
    hy::ws_record_init(buf + 1024, 1024, B);
    CHECK(hy::ws_record_use(buf, 1024, A));
    CHECK(hy::ws_record_use(buf + 1024, 1024, B));
    // using a workspace drops other plans' records that its bytes overlap
    CHECK(hy::ws_record_use(buf, 1536, A) == true);
    CHECK(!hy::ws_record_use(buf + 1024, 1024, B));
    hy::ws_record_drop(A);
    CHECK(hy::ws_record_count() == 0);
    // many threads recording and dropping at once
    std::vector<std::thread> th;
    static char big[64 * 4096];
    for (int t = 0; t < 8; ++t)
        th.emplace_back([t] {
            for (int i = 0; i < 2000; ++i) {
                char* w = big + (size_t)((t * 8 + i % 8) * 4096);
                const uint64_t tok = 5000 + (uint64_t)t;
                hy::ws_record_init(w, 4096, tok);
                if (!hy::ws_record_use(w, 4096, tok)) ++g_fail;
                hy::ws_record_release(w, tok);
            }
        });
    for (auto& x : th) x.join();
    CHECK(hy::ws_record_count() == 0);
    printf("workspace record: ok\n");
}

int main()
{
    plans();
    workspace_record();
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("host checks passed\n");
    return 0;
}
