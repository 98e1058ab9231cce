// bpw_gemv_tile.h - the grouped batch-1 GEMV's tile (device code shared by the bit-serial kernel in
// bpw_gemv.hip and the byte-lane kernel in bpw_bytelane.hip; not part of the ABI). The two kernels run
// the same tiles, activation staging, two-set prefetch loop, reduction and output pass; only the select
// differs (the BL template argument): the bit-serial select of bpw_gemv.hip's header on activation bit
// planes, or the byte-lane select on the activation bytes themselves.
#pragma once

#include "bpw_device.h"

namespace bpw {

// ------------------------------------------------------------------------------------------
// Batch-1 grouped GEMV. The host cuts every job's row-groups into tiles (one job each; wide ones first
// and narrow ones last on each XCD) and the grid has one workgroup of kWaves waves per tile; the
// hardware dispatcher hands tiles to compute units as earlier ones finish, so every compute unit
// streams until the whole list is done. Per tile the workgroup stages the job's activation in LDS
// (bit planes, or the bytes for the byte-lane select), then its waves claim row-groups from an LDS
// counter: a compute unit serves older waves
// first, and claiming keeps the younger ones from being left with a fixed share to finish last. A
// row is served by G = 2^glog consecutive lanes; lane g reads beats g, g+G, ... of its row (one wave
// load = G*16 contiguous bytes of each of 64/G rows), holding only those K beats in registers. Each
// wave keeps its next row-group's loads in flight while it reduces the current one. Loads past the
// matrix use an offset that the buffer range check answers with zeros, which also covers the
// partial last row-group.

// IntMlp epilogue of one row of a gate/up pair (Tritium paper, "Numerics", IntMlp): the exact
// sums a_g, a_u become t = relu(a_g)^2 * a_u in 64-bit integers (|a| <= 128 * cols and the host
// admits cols <= 16383, so t cannot overflow).
__device__ __forceinline__ void write_pair_row(const DevJob &J, int row, int32_t ag, int32_t au) {
    if (J.out_i32) J.out_i32[row] = ag;
    if (J.out_up_i32) J.out_up_i32[row] = au;
    const int64_t g = ag > 0 ? (int64_t)ag : 0;
    J.t_out[row] = (g * g) * (int64_t)au;
}

// K = S_g^2 * S_u in float64, S = x_scale * w_scale (exact products of two floats); written by one
// thread of the pair's first tile.
__device__ __forceinline__ void write_pair_k(const DevJob &J) {
    const double xs = (double)job_x_scale(J);
    const double sg = xs * (double)J.w_scale, su = xs * (double)J.w_scale_up;
    *J.k_out = (sg * sg) * su;
}

// Row sums collect in LDS (sums[], one slot per row of the tile) and leave in one coalesced pass
// at the end: a vector store inside the streaming loop would count against the same vector-memory
// counter as the weight loads.
// GLOG >= 0 and NB > 0 fix the geometry at compile time (one pass, NB == bpr); otherwise it is read
// from the job. A tile reduces the row-groups v = 0 .. V-1 of its own numbering: row-group u0 + v of
// the job's matrix, or for an IntMlp pair, row-groups u0 .. u1-1 of the gate (v < n) and then the
// same ones of the up projection (v >= n), whose sums land after the gate's in LDS. The pair is a
// run-time (wave-uniform) property, not a template argument: one copy of each streaming loop per
// geometry keeps the compiler's load-count waits exact (with a second copy of the loops in the
// kernel they fell back to waiting for every load in flight).
// The select of one row over the K beats a lane holds: bit-serial on activation bit planes, or
// byte-lane on the activation bytes (both staged in the same LDS slots).
template <bool BL, int K, int GLOG>
__device__ __forceinline__ int32_t select_partial(const u32x4 *xl, const u32x4 (&B)[K], int g, int G) {
    if constexpr (BL)
        return row_partial_bytelane<K, GLOG>(xl, B, g, G);
    else
        return row_partial<K, GLOG>(xl, B, g, G);
}

// The streaming part reads the job's fields from the tile record T (copies the host wrote); the job
// record J is read for the generic geometry and the output pass only, so its load overlaps the first
// beats.
template <bool BL, int K, int GLOG, int NB>
__device__ __forceinline__ void bs_tile(const Tile &T, const DevJob &J, int wave, int lane, u32x4 *xl,
                                           int32_t *sums, uint32_t *claim) {
    const int u0 = T.u0, u1 = T.u1;
    const int glog = GLOG >= 0 ? GLOG : J.glog;
    const int G = 1 << glog;
    const int g = lane & (G - 1);
    const int q = lane >> glog;
    const int rpi = 64 >> glog;
    const int bpr = NB > 0 ? NB : T.bpr;
    const int pass_blocks = K * G;
    const int nchunk = NB > 0 ? 1 : J.nchunk;
    const bool pair = T.pair != 0;
    const int n = u1 - u0;
    const int V = pair ? 2 * n : n;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(T.planes, T.plane_bytes);
    const __amdgpu_buffer_rsrc_t wu = make_rsrc(pair ? T.planes_up : T.planes, T.plane_bytes);
    // Row-group v's beats (v is wave-uniform, so the matrix choice is a scalar select).
    auto issue = [&](u32x4 (&B)[K], int v, int bb) {
        const bool up = v >= n;
        const int u = u0 + (up ? v - n : v);
        issue_row<K, NB>(B, up ? wu : wr, (uint32_t)(u * rpi + q), v < V, bb, G, bpr);
    };
    // The output pass's job fields, read once the first beats are out (the empty asm keeps the compiler
    // from waiting for them before those beats, and from reloading them after the last barrier, where
    // each load stood before the tile's stores).
    int32_t rows = 0;
    int32_t *out_i32 = nullptr;
    float *out_f32 = nullptr;
    const float *xs_ptr = nullptr;
    float xs = 0.f, w_scale = 0.f;
    for (int ch = 0; ch < nchunk; ++ch) {
        const int b0 = ch * pass_blocks;
        const int nb = min(pass_blocks, bpr - b0);
        const int bb = b0 + g;
        u32x4 B0[K], B1[K];
        int v = wave;  // every wave's first row-group is fixed; the rest are claimed
        issue(B0, v, bb);
        if (ch == 0) {
            rows = J.rows;
            out_i32 = J.out_i32;
            out_f32 = J.out_f32;
            w_scale = J.w_scale;
            xs = J.x_scale;
            xs_ptr = J.x_scale_ptr;  // dereferenced at the output pass: a vector load waited for here
                                     // would wait for the beats in flight too
            asm volatile("" : "+s"(rows), "+s"(out_i32), "+s"(out_f32), "+s"(w_scale), "+s"(xs), "+s"(xs_ptr));
        }
        __syncthreads();  // every wave is done with the previous planes, sums and counter
        if (threadIdx.x == 0) *claim = (uint32_t)kWaves;
        if constexpr (BL)
            stage_bytes(xl, T.x, b0, nb, wave, lane);
        else
            stage_planes(xl, T.x, b0, nb, wave, lane);
        __syncthreads();
        // Two register sets alternate: the loads of the next row-group leave before the current one
        // is reduced. One trip handles two row-groups with no exit in between, so every load is
        // issued on every path (row-groups past V read zeros and store nothing) and the compiler's
        // waits cover exactly the older set.
        while (v < V) {
            const int va = claim_next(claim, lane);
            issue(B1, va, bb);
            asm volatile("" ::: "memory");
            {
                const int32_t tot = group_sum(select_partial<BL, K, GLOG>(xl, B0, g, G), glog);
                const int i = v * rpi + q;
                if (g == 0) sums[i] = ch == 0 ? tot : sums[i] + tot;  // passes are separated by barriers
            }
            const int vb = claim_next(claim, lane);
            issue(B0, vb, bb);
            asm volatile("" ::: "memory");
            {
                const int32_t tot = group_sum(select_partial<BL, K, GLOG>(xl, B1, g, G), glog);
                const int i = va * rpi + q;
                if (g == 0 && va < V) sums[i] = ch == 0 ? tot : sums[i] + tot;
            }
            v = vb;
        }
    }
    __syncthreads();
    const int row0 = u0 * rpi, nr = n * rpi;
    if (pair) {
        for (int i = threadIdx.x; i < nr; i += kThreads)
            if (row0 + i < J.rows) write_pair_row(J, row0 + i, sums[i], sums[nr + i]);
        if (u0 == 0 && threadIdx.x == 0) write_pair_k(J);
    } else {
        if (xs_ptr) xs = *xs_ptr;  // the job's activation scale from device memory
        for (int i = threadIdx.x; i < nr; i += kThreads) {
            const int row = row0 + i;
            if (row < rows) {
                const int32_t sum = sums[i];
                out_i32[row] = sum;
                if (out_f32) out_f32[row] = ((float)sum * xs) * w_scale;  // each product rounded on its own
            }
        }
    }
}

// cols == 0: every row is the empty sum (row-groups of 64 rows).
__device__ __forceinline__ void bs_tile_empty(const DevJob &J, int u0, int u1, int wave, int lane) {
    for (int u = u0 + wave; u < u1; u += kWaves) {
        const int row = u * 64 + lane;
        if (row < J.rows) {
            if (J.pair)
                write_pair_row(J, row, 0, 0);
            else
                write_row(J, job_x_scale(J), row, 0);
        }
    }
    if (J.pair && u0 == 0 && threadIdx.x == 0) write_pair_k(J);
}

template <bool BL>
__device__ __forceinline__ void bs_dispatch(const DevJob &J, const Tile &t, int wave, int lane, u32x4 *xl,
                                            int32_t *sums, uint32_t *claim) {
    if (t.bpr == 40)  // 2560-column rows: 8 lanes x 5 beats
        bs_tile<BL, 5, 3, 40>(t, J, wave, lane, xl, sums, claim);
    else if (t.bpr == 108)  // 6912-column rows: 32 lanes x 4 beats (108 of 128 used)
        bs_tile<BL, 4, 5, 108>(t, J, wave, lane, xl, sums, claim);
    else if (t.bpr == 0)
        bs_tile_empty(J, t.u0, t.u1, wave, lane);
    else if (J.kblk == 1)
        bs_tile<BL, 1, -1, 0>(t, J, wave, lane, xl, sums, claim);
    else
        bs_tile<BL, 2, -1, 0>(t, J, wave, lane, xl, sums, claim);
}


}  // namespace bpw
