// host_check.cpp -- drives the host side of libssd (problem checks, the launch planner,
// workspace sizing, the plan description and the argument validation of every entry
// point) over a grid of shapes, edge values included, without any device work.  It is
// built together with ssd_api.hip under AddressSanitizer and UndefinedBehaviorSanitizer
// (host code only) and run on a machine without a GPU: every call below must return
// before its first HIP call, and a sanitizer report or a wrong status fails the run.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "ssd.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, const ssd_problem& p) {
    if (ok) return;
    ++failures;
    std::fprintf(stderr, "FAIL %s: b=%lld T=%lld H=%lld P=%lld N=%lld G=%lld Q=%lld nseq=%lld dtype=%d\n", what,
                 (long long)p.batch, (long long)p.seqlen, (long long)p.nheads, (long long)p.headdim,
                 (long long)p.dstate, (long long)p.ngroups, (long long)p.chunk_len, (long long)p.nseq, p.dtype);
}

// fake device addresses, 4 TiB apart (more than any array of the problems below),
// 256-byte aligned: never dereferenced
void* fake(int k) { return reinterpret_cast<void*>((uintptr_t)k << 42); }

// every host-only query on one problem, and calls of the entry points that must fail
// validation before any device work
void exercise(const ssd_problem& p) {
    const int rc = ssd_check_problem(&p);
    const size_t ws = ssd_workspace_bytes(&p);
    expect((rc == SSD_OK) == (ws > 0), "workspace bytes iff the problem is valid", p);
    char buf[256];
    for (size_t len : {(size_t)1, (size_t)7, sizeof buf}) {
        std::memset(buf, 'x', sizeof buf);
        const int drc = ssd_plan_describe(&p, buf, len);
        expect(drc == rc, "describe status", p);
        expect(std::memchr(buf, 0, len) != nullptr, "describe NUL-terminated within len", p);
        if (len < sizeof buf) expect(buf[len] == 'x', "describe writes at most len bytes", p);
    }
    if (rc == SSD_OK) {
        std::memset(buf, 0, sizeof buf);
        ssd_plan_describe(&p, buf, sizeof buf);
        expect(std::strncmp(buf, "walk=", 5) == 0 && std::strstr(buf, ";prep=") && std::strstr(buf, ";summary="),
               "describe format", p);
    }
    const size_t bws = ssd_backward_workspace_bytes(&p);
    if (rc != SSD_OK) expect(bws == 0, "no backward workspace for an invalid problem", p);
    if (bws) expect(bws >= ws, "backward workspace covers the forward's", p);

    const bool packed = p.nseq != p.batch;
    const void* off = packed ? fake(6) : nullptr;
    // a required pointer missing: invalid argument (or the problem's own status)
    const int want = rc == SSD_OK ? SSD_ERR_INVALID_ARG : rc;
    int r = ssd_forward(&p, nullptr, (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off, fake(7),
                        (float*)fake(8), fake(9), ws, nullptr);
    expect(r == want, "forward without X", p);
    r = ssd_forward_stage(1, &p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off,
                          nullptr, (float*)fake(8), fake(9), ws, nullptr);
    expect(r == want, "prep stage without Y", p);
    // misaligned X
    r = ssd_forward(&p, (const char*)fake(1) + 4, (const float*)fake(2), fake(3), fake(4), nullptr,
                    (const int32_t*)off, fake(7), (float*)fake(8), fake(9), ws, nullptr);
    expect(r == want, "forward with misaligned X", p);
    // Y on top of X, and the workspace on top of B
    r = ssd_forward(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off, fake(1),
                    (float*)fake(8), fake(9), ws, nullptr);
    expect(r == want, "forward with Y aliasing X", p);
    r = ssd_forward(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off, fake(7),
                    (float*)fake(8), fake(3), ws, nullptr);
    expect(r == want, "forward with the workspace aliasing B", p);
    if (rc == SSD_OK && ws > 256) {
        r = ssd_forward(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off, fake(7),
                        (float*)fake(8), fake(9), ws - 256, nullptr);
        expect(r == SSD_ERR_WORKSPACE, "forward with a small workspace", p);
    }
    if (rc == SSD_OK && ws > SSD_NOALLOC_SCRATCH_BYTES) {
        r = ssd_forward_noalloc(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off,
                                fake(7), (float*)fake(8), nullptr);
        expect(r == SSD_ERR_TOO_LARGE, "no-allocation forward beyond its scratch", p);
    }
    if (rc != SSD_OK) {
        r = ssd_forward_noalloc(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off,
                                fake(7), (float*)fake(8), nullptr);
        expect(r == rc, "no-allocation forward of an invalid problem", p);
    }
    // backward: dX missing; dX on top of dY
    r = ssd_backward(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off, fake(5),
                     nullptr, fake(10), nullptr, nullptr, (float*)fake(12), fake(13), fake(14), nullptr, fake(15), bws,
                     nullptr);
    expect(r == (bws ? SSD_ERR_INVALID_ARG : r), "backward without dX", p);
    if (bws) {
        r = ssd_backward(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off, fake(5),
                         nullptr, fake(10), nullptr, fake(10), (float*)fake(12), fake(13), fake(14), nullptr, fake(15),
                         bws, nullptr);
        expect(r == SSD_ERR_INVALID_ARG, "backward with dX aliasing dY", p);
        r = ssd_backward(&p, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, (const int32_t*)off, fake(5),
                         nullptr, fake(10), nullptr, fake(11), (float*)fake(12), fake(13), fake(14), nullptr, fake(1),
                         bws, nullptr);
        expect(r == SSD_ERR_INVALID_ARG, "backward with the workspace aliasing X", p);
    }
    // decode: the problem of one step per sequence, with y missing
    ssd_problem d = p;
    d.seqlen = 1;
    d.nseq = d.batch;
    r = ssd_decode_step(&d, fake(1), (const float*)fake(2), fake(3), fake(4), (float*)fake(5), nullptr, nullptr);
    expect(r != SSD_OK, "decode without y", d);
}

}  // namespace

int main() {
    const int64_t big = (int64_t)1 << 40, huge = INT64_MAX;
    const int64_t batches[] = {1, 2, 7, 0, -3, big, huge};
    const int64_t seqlens[] = {1, 31, 300, 4096, (int64_t)1 << 20, 0, big, huge};
    const int64_t heads[] = {1, 3, 8, 80, 0, big};
    const int64_t dims[] = {16, 32, 48, 64, 128, 256, 40, 512, 0, huge};
    const int64_t groups[] = {1, 2, 80, 0, big};
    const int64_t chunks[] = {16, 64, 100, 256, 512, 0};
    const int dtypes[] = {SSD_DTYPE_F32, SSD_DTYPE_BF16, 5};
    long n = 0;
    for (int64_t b : batches)
        for (int64_t T : seqlens)
            for (int64_t H : heads)
                for (int64_t P : dims)
                    for (int64_t N : dims)
                        for (int64_t G : groups)
                            for (int64_t Q : chunks)
                                for (int dt : dtypes)
                                    for (int varlen = 0; varlen < 2; ++varlen) {
                                        // keep the grid to a few hundred thousand problems
                                        if ((P != 64 && N != 128 && Q != 256) || (G != 1 && H < 3 && G != 0))
                                            continue;
                                        ssd_problem p;
                                        p.batch = varlen ? 1 : b;
                                        p.seqlen = T;
                                        p.nheads = H;
                                        p.headdim = P;
                                        p.dstate = N;
                                        p.ngroups = G;
                                        p.chunk_len = Q;
                                        p.nseq = varlen ? (b > 0 && b < 100 ? 3 * b : b) : b;
                                        p.dtype = dt;
                                        p.reserved = 0;
                                        exercise(p);
                                        ++n;
                                    }
    // null problem and null buffers
    expect(ssd_check_problem(nullptr) == SSD_ERR_INVALID_ARG, "null problem", ssd_problem{});
    expect(ssd_workspace_bytes(nullptr) == 0, "null problem workspace", ssd_problem{});
    char c = 'x';
    ssd_problem ok{2, 300, 4, 64, 128, 2, 64, 2, SSD_DTYPE_BF16, 0};
    expect(ssd_plan_describe(&ok, nullptr, 8) == SSD_ERR_INVALID_ARG, "describe into NULL", ok);
    expect(ssd_plan_describe(&ok, &c, 0) == SSD_ERR_INVALID_ARG && c == 'x', "describe with len 0", ok);
    ok.reserved = 1;
    expect(ssd_check_problem(&ok) == SSD_ERR_INVALID_ARG, "reserved field set", ok);
    for (int s = -8; s <= 2; ++s) expect(ssd_status_string(s) != nullptr, "status string", ok);
    expect(ssd_abi_version() == SSD_ABI_VERSION, "abi version", ok);
    std::printf("host check: %ld problems, %d failures\n", n, failures);
    return failures ? 1 : 0;
}
