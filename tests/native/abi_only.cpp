// End-to-end use of libddp through its C ABI alone: HIP allocations and
// streams, plain pointers, no Python and no torch.
//
// The inputs are dyadic (x = (w + 1) * m / 64 with m in 1..7) and W is a power
// of two, so every term x * fp32(1/W) and every partial sum of the fold is
// exact: the reduced value is the exact mean, whatever the fold order,
// (W + 1) / 2 * m / 64. That closed form is the check here; the bit-exact
// comparison against the CPU oracle is the Python tests' job.
//
// With unused-parameter detection (third argument 1) replica w uses gradient
// p unless (w + p) % 3 == 0, and gradient 2 is used by no replica. A used
// gradient's value is then S_p * m / (64 W), S_p the sum of w + 1 over the
// replicas that used it (the others contribute zeros), still exact; gradient
// 2's flat slice must keep its contents.
//
// usage: abi_only W collective [unused]   (W a power of two, collective 0 or 1)
// exit status 0 when every element of every replica matches.
#include "ddp.h"

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#define HIP_OK(x)                                                                       \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            std::exit(2);                                                               \
        }                                                                               \
    } while (0)

#define DDP_OK_(x)                                                                      \
    do {                                                                                \
        int rc_ = (x);                                                                  \
        if (rc_ != DDP_OK) {                                                            \
            std::fprintf(stderr, "%s: %d %s\n", #x, rc_, ddp_last_error());             \
            std::exit(2);                                                               \
        }                                                                               \
    } while (0)

static float input_value(int w, int64_t i)
{
    return float((w + 1) * int(i % 7 + 1)) / 64.0f;
}

int main(int argc, char **argv)
{
    const int W = argc > 1 ? std::atoi(argv[1]) : 8;
    const int collective = argc > 2 ? std::atoi(argv[2]) : DDP_ALL_REDUCE;
    const int unused = argc > 3 ? std::atoi(argv[3]) : 0;
    if (W < 1 || (W & (W - 1)) != 0 || W > 64) {
        std::fprintf(stderr, "W must be a power of two up to 64\n");
        return 2;
    }
    const int32_t kUnusedEverywhere = 2;
    // gradient sizes in elements, in registration order: odd sizes, a
    // zero-size gradient and one larger than a tile
    const std::vector<int64_t> numel = {1000, 4096, 77, 0, 100003, 3, 65536, 1};
    const int32_t P = int32_t(numel.size());
    std::vector<int64_t> bytes(P);
    for (int p = 0; p < P; ++p) bytes[p] = 4 * numel[p];

    std::vector<int32_t> bucket_of(P), bucket_params(P), bucket_nparams(P);
    std::vector<int64_t> offset(P), bucket_bytes(P);
    int32_t B = 0;
    DDP_OK_(ddp_plan_buckets(P, bytes.data(), nullptr, DDP_ORDER_REVERSE, 64 << 10, 16 << 10, bucket_of.data(),
                             offset.data(), bucket_params.data(), bucket_nparams.data(), bucket_bytes.data(), &B));
    int64_t total = 0;   // flat elements per replica
    std::vector<int64_t> bucket_start(B);
    for (int b = 0; b < B; ++b) {
        bucket_start[b] = total;
        total += bucket_bytes[b] / 4;
    }

    // replica w's gradients (device) and flat buffer (device)
    std::vector<void *> grads(size_t(W) * P, nullptr);
    std::vector<float *> flat(W, nullptr);
    for (int w = 0; w < W; ++w) {
        for (int p = 0; p < P; ++p) {
            if (numel[p] == 0) continue;
            HIP_OK(hipMalloc(&grads[size_t(w) * P + p], bytes[p]));
            std::vector<float> h(numel[p]);
            for (int64_t i = 0; i < numel[p]; ++i) h[i] = input_value(w, i);
            HIP_OK(hipMemcpy(grads[size_t(w) * P + p], h.data(), bytes[p], hipMemcpyHostToDevice));
        }
        HIP_OK(hipMalloc(&flat[w], 4 * total));
        HIP_OK(hipMemset(flat[w], 0xFF, 4 * total));   // NaN pattern: any slot left unwritten shows
    }
    hipStream_t compute = nullptr, comm = nullptr;
    HIP_OK(hipStreamCreate(&compute));
    HIP_OK(hipStreamCreate(&comm));

    ddp_reducer_desc d{};
    d.world = W;
    d.n_params = P;
    d.param_numel = numel.data();
    d.bucket_of = bucket_of.data();
    d.offset_in_bucket = offset.data();
    d.n_buckets = B;
    d.input_mode = DDP_IN_F32_COPY;
    d.grads = grads.data();
    d.flat = flat.data();
    d.compute_stream = compute;
    d.comm_stream = comm;
    d.collective = collective;
    d.find_unused = unused;
    d.workspace_bytes = ddp_workspace_bytes(&d);
    if (d.workspace_bytes == 0) {
        std::fprintf(stderr, "ddp_workspace_bytes: %s\n", ddp_last_error());
        return 2;
    }
    HIP_OK(hipMalloc(&d.workspace, d.workspace_bytes));
    ddp_reducer *r = nullptr;
    DDP_OK_(ddp_reducer_create(&d, &r));

    // used[w * P + p]: replica w produced gradient p (unused detection only)
    std::vector<uint8_t> used(size_t(W) * P, 1);
    std::vector<int64_t> used_sum(P, int64_t(W) * (W + 1) / 2);   // S_p: sum of w + 1 over users
    if (unused) {
        for (int p = 0; p < P; ++p) {
            used_sum[p] = 0;
            for (int w = 0; w < W; ++w) {
                const bool u = p != kUnusedEverywhere && (w + p) % 3 != 0;
                used[size_t(w) * P + p] = u;
                if (u) used_sum[p] += w + 1;
            }
        }
    }
    std::vector<int32_t> order;   // gradients someone used, in reverse registration order
    for (int i = P - 1; i >= 0; --i)
        if (used_sum[i] > 0) order.push_back(i);
    const int32_t n_marks = int32_t(order.size());
    int64_t bad = 0;
    for (int iter = 0; iter < 2; ++iter) {
        DDP_OK_(ddp_prepare_for_backward(r));
        if (unused) DDP_OK_(ddp_set_local_used(r, used.data()));
        int32_t done = 0;
        DDP_OK_(ddp_mark_ready_many(r, order.data(), n_marks, &done));
        DDP_OK_(ddp_finish(r, 1));
        int32_t launched = 0;
        DDP_OK_(ddp_get_launched(r, &launched));
        if (done != n_marks || launched != B) {
            std::fprintf(stderr, "marked %d of %d, launched %d of %d buckets\n", done, n_marks, launched, B);
            return 1;
        }
        for (int w = 0; w < W; ++w) {
            std::vector<float> got(total);
            HIP_OK(hipMemcpy(got.data(), flat[w], 4 * total, hipMemcpyDeviceToHost));
            for (int p = 0; p < P; ++p) {
                const int b = bucket_of[p];
                const int64_t n = bucket_bytes[b] / 4, q = (n + W - 1) / W;
                const int64_t base = bucket_start[b] + offset[p] / 4;
                for (int64_t i = 0; i < numel[p]; ++i) {
                    const int64_t e = offset[p] / 4 + i;   // element of the bucket
                    const bool owned = collective == DDP_ALL_REDUCE || e / q == w;
                    if (!owned) continue;                    // another replica's shard: never written
                    if (used_sum[p] == 0) {                  // used by no replica: never written
                        uint32_t bits;
                        std::memcpy(&bits, &got[base + i], 4);
                        if (bits != 0xFFFFFFFFu && bad++ < 5)
                            std::fprintf(stderr, "replica %d unused gradient %d element %lld was written\n", w,
                                         p, (long long)i);
                        continue;
                    }
                    const float want = float(used_sum[p]) * float(i % 7 + 1) / (64.0f * float(W));
                    if (got[base + i] != want && bad++ < 5)
                        std::fprintf(stderr, "replica %d gradient %d element %lld: %g, want %g\n", w, p,
                                     (long long)i, double(got[base + i]), double(want));
                }
            }
        }
    }
    DDP_OK_(ddp_reducer_destroy(r));
    HIP_OK(hipStreamDestroy(compute));
    HIP_OK(hipStreamDestroy(comm));
    for (void *g : grads)
        if (g) HIP_OK(hipFree(g));
    for (float *f : flat) HIP_OK(hipFree(f));
    HIP_OK(hipFree(d.workspace));
    if (bad) {
        std::fprintf(stderr, "%lld mismatches\n", (long long)bad);
        return 1;
    }
    std::printf("abi_only ok: W=%d collective=%d unused=%d, %d gradients, %d buckets, %lld elements, 2 iterations\n",
                W, collective, unused, P, B, (long long)total);
    return 0;
}
