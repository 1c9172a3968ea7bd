// spec_sample.hip -- speculative-sampling acceptance (rejection sampling) on
// MI355X (gfx950), the step after the verify pass.
//
// The operation is defined in include/paged_attn.h (paged_attn_rejection_sample).
// Sources: "Latency and cost in production" §10.6.2 (a draft token passes
// when p >= q and otherwise with probability p/q; after a rejection the
// replacement comes from norm(max(0, p - q)); when every draft passes, the
// target's extra position gives a bonus token) and "Speculative decoding
// principles" (7.2.1), acceptance rule and residual distribution (the test is
// one uniform u with u < p/q; the residual is a transient distribution
// computed at the rejected position only).
//
// Design: the work is one pass over one vocabulary row per sequence (the
// residual's p and q rows, or the bonus row), so it is HBM-bound; the rest is
// K scalar lookups.  Two kernels:
//  * pass 1, one wave per (4096-entry chunk of the row, sequence): finds the
//    first rejection (one lane per draft, a wave ballot); each lane loads 64
//    consecutive entries straight into registers (16-byte loads, all in flight
//    at once; plain rather than non-temporal, so that the wave's 16-byte
//    pieces of one cache line meet in L1) and the wave writes the chunk's sums
//    of the sampling weights and of p, in binary64;
//  * pass 2, one wave per sequence: folds the chunk sums, finds the chunk in
//    which the running sum first exceeds u * total, re-reads that chunk only
//    and finds the token inside it.
// Every sum has one fixed association, the same in both passes: 64 entries
// per lane left to right, then the 64 lane totals left to right, then the
// chunk totals left to right.  The running sum is therefore non-decreasing
// over the whole row, ends at the total that the target was taken from, and
// only rises on entries of positive weight, so a zero-weight token is never
// drawn.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "paged_attn.h"
#include "status.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kLanes = 64;                     // one wave
constexpr int kPerLane = 64;                   // consecutive entries held and summed by one lane
constexpr int kChunk = kLanes * kPerLane;      // vocabulary entries per chunk (one wave)
constexpr int kMaxDrafts = kLanes;
constexpr int kMaxChunks = 256;                // vocabulary up to 1,048,576

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct SampleArgs {
    const float* p;          // [B][K+1][V]
    const float* q;          // [B][K][V]
    const int32_t* draft;    // [B][K]
    const float* u_accept;   // [B][K]
    const float* u_sample;   // [B]
    int32_t* tokens;         // [B][K+1]
    int32_t* accepted;       // [B]
    double* chunk_sums;      // [B][chunks][2]: sampling weights, p
    int32_t* first_rej;      // [B]: index of the first rejected draft (K if none)
    int32_t K, V, chunks;
    int32_t vec4;            // rows are 16-byte aligned (V % 4 == 0, aligned bases)
};

// Index of the first rejected draft of sequence b (K if all pass), in every
// lane of the calling wave.  Draft i passes iff u * q(x) < p(x), exact in
// binary64 (both factors carry 24-bit significands).
__device__ __forceinline__ int first_rejection(const SampleArgs& a, int b, int lane)
{
    bool rejected = false;
    if (lane < a.K) {
        const int64_t di = (int64_t)b * a.K + lane;
        const int x = min(max(a.draft[di], 0), a.V - 1);
        const float px = a.p[((int64_t)b * (a.K + 1) + lane) * a.V + x];
        const float qx = a.q[di * a.V + x];
        rejected = !((double)a.u_accept[di] * (double)qx < (double)px);
    }
    const uint64_t m = __ballot(rejected);
    return m ? __ffsll((unsigned long long)m) - 1 : a.K;
}

__device__ __forceinline__ double weight(float pv, float qv, bool residual)
{
    if (!residual) return (double)pv;
    const double d = (double)pv - (double)qv;
    return d > 0.0 ? d : 0.0;
}

// Entries [j0, j0 + 64) of a row into registers (0 past the end of the row);
// all loads are issued before any is used.
template <bool NT>
__device__ __forceinline__ void load_run(const float* row, int j0, int V, bool vec4,
                                         float (&x)[kPerLane])
{
    if (vec4 && j0 + kPerLane <= V) {
        const f32x4* s = reinterpret_cast<const f32x4*>(row + j0);
#pragma unroll
        for (int i = 0; i < kPerLane / 4; ++i) {
            const f32x4 v = NT ? __builtin_nontemporal_load(s + i) : s[i];
            x[4 * i] = v.x;
            x[4 * i + 1] = v.y;
            x[4 * i + 2] = v.z;
            x[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int j = j0 + i;
            const float v = row[min(j, V - 1)];
            x[i] = j < V ? v : 0.f;
        }
    }
}

// Left-to-right binary64 sums of a lane's 64 entries: sampling weights and p.
__device__ __forceinline__ void run_sums(const float (&xp)[kPerLane], const float (&xq)[kPerLane],
                                         bool residual, double& w_sum, double& p_sum)
{
    double sw = 0.0, s_p = 0.0;
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) {
        sw += weight(xp[k], xq[k], residual);
        s_p += (double)xp[k];
    }
    w_sum = sw;
    p_sum = s_p;
}

// Rows of sequence b at position r: p, and q when r is a rejected draft.
__device__ __forceinline__ const float* p_row(const SampleArgs& a, int b, int r)
{
    return a.p + ((int64_t)b * (a.K + 1) + r) * a.V;
}
__device__ __forceinline__ const float* q_row(const SampleArgs& a, int b, int r)
{
    return a.q + ((int64_t)b * a.K + r) * a.V;
}

// Pass 1: one wave per (chunk, sequence); writes the chunk's sums.
__global__ __launch_bounds__(kLanes) void spec_sample_chunks(SampleArgs a)
{
    __shared__ double tot[2][kLanes];
    const int c = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int r = first_rejection(a, b, lane);
    const bool residual = r < a.K;
    const int j0 = c * kChunk + lane * kPerLane;
    float xp[kPerLane], xq[kPerLane];
    load_run<false>(p_row(a, b, r), j0, a.V, a.vec4, xp);
    if (residual) {
        load_run<false>(q_row(a, b, r), j0, a.V, a.vec4, xq);
    } else {
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) xq[k] = 0.f;
    }
    run_sums(xp, xq, residual, tot[0][lane], tot[1][lane]);
    __syncthreads();
    if (lane == 0) {
        double s0 = 0.0, s1 = 0.0;
#pragma unroll
        for (int l = 0; l < kLanes; ++l) {
            s0 += tot[0][l];
            s1 += tot[1][l];
        }
        double* out = a.chunk_sums + ((int64_t)b * a.chunks + c) * 2;
        out[0] = s0;
        out[1] = s1;
        if (c == 0) a.first_rej[b] = r;
    }
}

// Pass 2: one wave per sequence; picks the chunk, then the token inside it.
__global__ __launch_bounds__(kLanes) void spec_sample_pick(SampleArgs a)
{
    __shared__ double sums[2][kMaxChunks];     // chunk sums, then their running sums
    __shared__ double tot[2][kLanes];
    __shared__ double lane_base[kLanes];
    __shared__ double s_total[2];
    const int b = blockIdx.x, lane = threadIdx.x;
    // everything this wave needs from pass 1 and the inputs, in one round trip
    const int r = a.first_rej[b];
    const float u = a.u_sample[b];
    const int32_t my_draft = lane < a.K ? a.draft[(int64_t)b * a.K + lane] : -1;
    for (int c = lane; c < a.chunks; c += kLanes) {
        const double* in = a.chunk_sums + ((int64_t)b * a.chunks + c) * 2;
        sums[0][c] = in[0];
        sums[1][c] = in[1];
    }
    __syncthreads();
    if (lane == 0) {
        // running sums over the chunks, left to right (the association pass 1 used)
        double t0 = 0.0, t1 = 0.0;
#pragma unroll 8
        for (int c = 0; c < a.chunks; ++c) {
            t0 += sums[0][c];
            t1 += sums[1][c];
            sums[0][c] = t0;
            sums[1][c] = t1;
        }
        s_total[0] = t0;
        s_total[1] = t1;
    }
    __syncthreads();
    // an empty residual falls back to p at the same position
    const int kind = s_total[0] > 0.0 ? 0 : 1;
    const double total = s_total[kind];
    const double target = (double)u * total;
    int chunk = -1;
    if (total > 0.0) {
        for (int c0 = 0; c0 < a.chunks; c0 += kLanes) {
            const int c = c0 + lane;
            const uint64_t m = __ballot(c < a.chunks && sums[kind][c] > target);
            if (m) {
                chunk = c0 + __ffsll((unsigned long long)m) - 1;
                break;
            }
        }
    }
    int32_t token = -1;
    if (chunk >= 0) {
        const double pex = chunk > 0 ? sums[kind][chunk - 1] : 0.0;
        const bool residual = r < a.K && kind == 0;
        const int j0 = chunk * kChunk + lane * kPerLane;
        float xp[kPerLane], xq[kPerLane];
        load_run<false>(p_row(a, b, r), j0, a.V, a.vec4, xp);
        if (residual) {
            load_run<false>(q_row(a, b, r), j0, a.V, a.vec4, xq);
        } else {
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) xq[k] = 0.f;
        }
        run_sums(xp, xq, residual, tot[0][lane], tot[1][lane]);
        __syncthreads();
        const int walk = residual ? 0 : 1;     // which sums the walk accumulates
        if (lane == 0) {
            double run = 0.0;
#pragma unroll
            for (int l = 0; l < kLanes; ++l) {
                lane_base[l] = run;
                run += tot[walk][l];
            }
        }
        __syncthreads();
        // running sum at entry k of this lane: pex + (lane_base + this lane's first k + 1)
        const double lb = lane_base[lane];
        int found = kPerLane;
        double run = 0.0;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            run += weight(xp[k], xq[k], residual);
            if (found == kPerLane && pex + (lb + run) > target) found = k;
        }
        const uint64_t m = __ballot(found < kPerLane);
        if (m) {
            const int first = __ffsll((unsigned long long)m) - 1;
            token = chunk * kChunk + first * kPerLane + __shfl(found, first);
        }
    }
    if (lane == 0) a.accepted[b] = r;
    for (int i = lane; i <= a.K; i += kLanes)     // i < r only for i == lane (r <= 64)
        a.tokens[(int64_t)b * (a.K + 1) + i] = i < r ? my_draft : i == r ? token : -1;
}

int chunks_for(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

}  // namespace

PA_API size_t paged_attn_rejection_sample_workspace_bytes(int32_t batch, int32_t vocab)
{
    if (batch < 1 || vocab < 1) return 0;
    return (size_t)batch * chunks_for(vocab) * 2 * sizeof(double) + (size_t)batch * sizeof(int32_t);
}

PA_API pa_status paged_attn_rejection_sample(const float* p, const float* q, const int32_t* draft,
                                             const float* u_accept, const float* u_sample,
                                             int32_t batch, int32_t num_drafts, int32_t vocab,
                                             int32_t* tokens, int32_t* num_accepted,
                                             void* workspace, size_t workspace_bytes, void* stream)
{
    if (!p || !u_sample || !tokens || !num_accepted)
        return pa_record_error(PA_ERR_INVALID_ARG, "null p, u_sample, tokens or num_accepted");
    if (num_drafts > 0 && (!q || !draft || !u_accept))
        return pa_record_error(PA_ERR_INVALID_ARG, "null q, draft or u_accept with num_drafts > 0");
    if (batch < 1 || vocab < 1 || num_drafts < 0)
        return pa_record_error(PA_ERR_INVALID_ARG, "batch and vocab must be >= 1, num_drafts >= 0");
    if (num_drafts > kMaxDrafts)
        return pa_record_error(PA_ERR_UNSUPPORTED, "at most 64 drafts per sequence");
    if (chunks_for(vocab) > kMaxChunks)
        return pa_record_error(PA_ERR_UNSUPPORTED, "vocabulary above 1,048,576 entries");
    if (batch > 65535) return pa_record_error(PA_ERR_UNSUPPORTED, "batch above 65535");
    const size_t need = paged_attn_rejection_sample_workspace_bytes(batch, vocab);
    if (!workspace || workspace_bytes < need)
        return pa_record_error(PA_ERR_WORKSPACE, "workspace missing or too small");
    if (reinterpret_cast<uintptr_t>(workspace) % alignof(double))
        return pa_record_error(PA_ERR_INVALID_ARG, "workspace must be 8-byte aligned");
    SampleArgs a;
    a.p = p;
    a.q = q;
    a.draft = draft;
    a.u_accept = u_accept;
    a.u_sample = u_sample;
    a.tokens = tokens;
    a.accepted = num_accepted;
    a.chunk_sums = static_cast<double*>(workspace);
    a.first_rej = reinterpret_cast<int32_t*>(a.chunk_sums + (size_t)batch * chunks_for(vocab) * 2);
    a.K = num_drafts;
    a.V = vocab;
    a.chunks = chunks_for(vocab);
    a.vec4 = vocab % 4 == 0 && reinterpret_cast<uintptr_t>(p) % 16 == 0 &&
             reinterpret_cast<uintptr_t>(q) % 16 == 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(spec_sample_chunks, dim3((unsigned)a.chunks, (unsigned)batch),
                       dim3(kLanes), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa_record_hip_error(e, "rejection sample pass 1 launch");
    hipLaunchKernelGGL(spec_sample_pick, dim3((unsigned)batch), dim3(kLanes), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return pa_record_hip_error(e, "rejection sample pass 2 launch");
    return PA_OK;
}
