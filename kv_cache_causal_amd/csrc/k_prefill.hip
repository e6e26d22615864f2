// K4: causal GQA prefill attention on the fp32 matrix cores (MFMA).
//
// "11 · Attention, vec ops, and the KV cache":
//   §2.1   out_t = sum_{s <= t} softmax(q_t . k_s * scale) v_s.
//   §2.4   query head h reads kv head h / (n_head / n_head_kv).
//   §3.2.4 token t's window is rows [0, pos[t]] of the layer's regions; positions are data
//          (any order, any gaps), so the mask is computed per (query, key) from pos.
//   §2.5   on a GPU the (query, key) matrix is tiled and the softmax runs online.
//
// Prefill is a dense contraction (a 4,096-token prompt with Qwen3-0.6B heads: >700 flop
// per byte), so both products run on v_mfma_f32_16x16x4_f32, full fp32 in and out.
// Design:
//   * Workgroup = 4 wave64s = 64 query rows of one kv head: GB heads of the kv group x TQ
//     tokens (GB * TQ = 64), so one K/V tile in LDS serves all of them.  Each wave owns 16
//     query rows (one head, 16 tokens).
//   * The transposed products keep every per-query quantity in one lane column:
//       S^T[key][q]  = K[key][:] . Q[q][:]       (A = K tile from LDS, B = Q in registers)
//       O^T[d][q]   += V^T[d][key] P^T[key][q]   (A = V tile from LDS, B = P in registers)
//     With lane l = 16 * g + c, the S^T accumulator of a 16-key block holds keys 4g..4g+3
//     of query c -- exactly the B operand the O^T product needs for its 4 k-steps, so P
//     never leaves registers.  The head-dim contraction of S^T is permuted so lane group
//     g owns dims [g*hd/4, (g+1)*hd/4): Q and K fragments are contiguous (b128 reads).
//   * Online softmax per query column: the row max is a max over 16 registers and two
//     cross-group lane swaps (no LDS); the rescale factor is per lane; the row sum stays
//     per lane group until the end.
//   * Causality from data: a block scans key tiles up to the max position of its tokens;
//     a wave skips tiles beyond its own max; the per-element mask (key > pos) is a select.
//   * Heavy query tiles (late positions) are launched first to shorten the tail.
//   * K and V tiles come into LDS by direct-to-LDS loads, each half of a tile while the
//     other half's products run: K(t+1)'s loads are issued once every wave has read K(t)
//     (they land during PV(t)), V(t+1)'s once every wave has read V(t) (they land during
//     S(t+1)).  No registers hold the tiles in flight and no LDS stores are issued for
//     them (staging through registers and LDS stores took a quarter of each tile's time
//     on a 4,096-token prompt, by per-tile timestamps, and was 2-4% slower).
//   * Short prompts give too few query tiles to fill 256 CUs, and each would walk its key
//     tiles one after another.  Then the host cuts every query tile's key range into
//     segments (same tile count each, the last one shorter); a workgroup scans one
//     segment and writes its unnormalised (m, l, O) record, and a merge kernel combines a
//     query's records by log-sum-exp (split-K, as for decode).
//   * Region formats: a binary16 window is widened, a Q8_0 window dequantized (scale *
//     code, exact in f32), once into an f32 copy that the f32 kernel reads, so the
//     products always see f32 values.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <vector>

#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}


template <int HD>
struct PrefillCfg {
    static constexpr int KT = prefill_key_tile(HD);  // keys per tile
    static constexpr int KB = KT / 16;              // 16-key blocks per tile
    static constexpr int DQ = HD / 4;               // dims per lane group
    // LDS row strides (floats): rows are unpadded, since the direct-to-LDS tile loads
    // write contiguous 1 KB pieces.  The K-fragment reads (16 rows, one column) are spread
    // over the banks by a swizzle instead (KSWZ below), which a bank-conflict probe on
    // gfx950 measured as good as 4 floats of padding; the V-fragment reads (contiguous row
    // pieces) are conflict-free unpadded.
    static constexpr int KSTR = HD;
    static constexpr int VSTR = HD;
    // K swizzle: 16-byte chunk c of tile row r sits at chunk position c ^ (r mod KSWZ),
    // KSWZ the largest power of two up to 16 that divides the row's HD / 4 chunks (so the
    // swizzle stays inside the row: 16 for head dims that are multiples of 64, 8 for 96
    // and 160, 4 for 80 and 112).
    static constexpr int KSWZ = (HD / 4) % 16 == 0 ? 16 : (HD / 4) % 8 == 0 ? 8
                              : (HD / 4) % 4 == 0 ? 4 : (HD / 4) % 2 == 0 ? 2 : 1;
    static constexpr int NDB = HD / 16;             // 16-dim output blocks
    // Output blocks fed by one V read: 4 when they group by 4, else 2 or 1.
    static constexpr int VEC = NDB % 4 == 0 ? 4 : NDB % 2 == 0 ? 2 : 1;
    static_assert(HD % 16 == 0 && (HD / 4) % KSWZ == 0 && NDB % VEC == 0, "head dim");
};

typedef int32_t intx4 __attribute__((ext_vector_type(4)));

// K/V tiles reach LDS by direct-to-LDS loads (global_load_lds_dwordx4: lane l's 16
// bytes land at the LDS address in M0 + 16 l; no registers hold them and no LDS store
// instructions are issued).  The load is written in inline assembly: the compiler's wait
// insertion treats every LDS read after such a load as depending on it and drains all
// loads in flight first, which would serialise the next tile's loads with this tile's
// reads.  The kernel waits for its own loads instead (wait_tile_dma), at points where
// only one tile's loads are outstanding.  M0 is saved and restored around the load (the
// kernel uses it nowhere else), with the wait states the hardware needs after writing it.
// The address is a uniform 64-bit base in SGPRs plus a 32-bit per-lane offset: one VGPR
// read per lane instead of two (the 64-bit per-lane form measured 4% slower on the
// 4,096-token prompt, the loads being issued while the other wave of the SIMD runs its
// MFMAs).
__device__ __forceinline__ void tile_dma16(const void *base, uint32_t off, uint32_t lds_base)
{
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %3\n\t"
                 "s_nop 1\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\t"
                 "s_nop 1\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(save)
                 : "v"(off), "s"(base), "s"(lds_base)
                 : "memory");
}
__device__ __forceinline__ void wait_tile_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Split-K record of one (segment, token, head): O[HD] unnormalised, then m (base 2), l and,
// in segment 0's record, the token's segment count.
template <int HD>
__device__ __forceinline__ float *part_record(const PrefillParams &p, int seg, int t, int h)
{
    return p.part + (((int64_t)seg * p.nt + t) * p.n_head + h) * (HD + 4);
}

template <int HD, typename KVT>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PrefillParams p, int32_t nblocks)
{
    static_assert(std::is_same<KVT, float>::value, "f32 tiles (other formats are widened first)");
    using C = PrefillCfg<HD>;
    constexpr int KT = C::KT, KB = C::KB, DQ = C::DQ, NDB = C::NDB, VEC = C::VEC;
    constexpr int KSTR = C::KSTR, VSTR = C::VSTR, F = C::KSWZ;
    constexpr int LD = KT * HD / (256 * 4);   // 1 KB loads per wave per tile (K or V)
    static_assert(LD * 256 * 4 == KT * HD && LD >= 1, "tile split");
    __shared__ __align__(16) float Ks[KT * KSTR];
    __shared__ __align__(16) float Vs[KT * VSTR];
    __shared__ int s_vbad;   // 1 once a tile of this block held a non-finite V value

    // XCD-aware mapping: consecutive workgroups go to the 8 XCDs in turn, so workgroup b
    // takes logical block (b % 8) * (nblocks / 8) + b / 8.  Each XCD then owns a
    // contiguous range of logical blocks -- one kv head's work units when the counts
    // divide -- and its L2 serves those units' shared K/V rows.  Within a range, heavy
    // (late-position) query tiles come first.
    const int GB = p.GB, TQ = p.TQ, n_hsub = p.n_hsub;
    const int per_xcd = (nblocks + 7) / 8;
    const int logical = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
    if (logical >= nblocks) return;
    const int hgroup = logical / p.units_per_hgroup;
    const int unit = logical - hgroup * p.units_per_hgroup;
    // Work unit (from the kernel arguments, or from device-visible memory for long
    // tables): a query tile, the key tiles [kt0, kt1) it scans, its segment index and the
    // tile's segment count, and the largest and smallest position among the tile's tokens
    // (computed on the host, so no workgroup reduces positions before its first load).
    intx4 ua, ub;
    if (p.units) {
        ua = reinterpret_cast<const intx4 *>(p.units)[2 * unit];
        ub = reinterpret_cast<const intx4 *>(p.units)[2 * unit + 1];
    } else {
        const int *u = p.iunits + unit * kUnitInts;
        ua = intx4{u[0], u[1], u[2], u[3]};
        ub = intx4{u[4], u[5], u[6], u[7]};
    }
    const int qtile = ua[0], kt0 = ua[1], kt1 = ua[1] + ua[2];
    const int seg = ua[3] >> 16, nseg = ua[3] & 0xffff;
    const int kmax = ub[0], kmin = ub[1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qc = lane & 15;   // query column of this lane
    const int grp = lane >> 4;  // lane group: key rows 4grp..4grp+3 of each 16-key block

    const int hk = hgroup / n_hsub;
    const int hs = hgroup - hk * n_hsub;
    const int G = p.n_head / p.n_head_kv;
    const int wpt = TQ / 16;                 // waves per head
    const int g = hs * GB + wave / wpt;      // head within the kv group
    const bool head_ok = g < G;
    const int h = hk * G + (head_ok ? g : 0);
    const int t = qtile * TQ + (wave % wpt) * 16 + qc;
    const bool tok_ok = t < p.nt;
    // This lane's position: contiguous prompts carry only the first one (no memory read
    // before the first tile's loads); other prompts read theirs.
    int pq = p.pos0 + t;
    if (p.pos) pq = p.pos[tok_ok ? t : 0];
    if (!tok_ok) pq = 0;

    s_vbad = 0;   // every thread, before the loop's first barrier orders it before any use
    const int nkt = p.n_head_kv * HD;
    const KVT *Kh = static_cast<const KVT *>(p.kc) + hk * HD;
    const KVT *Vh = static_cast<const KVT *>(p.vc) + hk * HD;

    // Tile staging: load j of wave w moves bytes [(w LD + j) 1024, +1024) of the K (V)
    // tile, lane l's 16 bytes at + 16 l, K rows swizzled (KSWZ).  Regions are padded to a
    // whole number of 64-row tiles (zero rows past the capacity, beyond every position and
    // so masked), so every tile row read is inside the region.
    constexpr int RBYTES = HD * 4;
    const uint32_t ks_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) float *)Ks) + wave * LD * 1024);
    const uint32_t vs_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) float *)Vs) + wave * LD * 1024);
    auto dma_k = [&](int key0) {
        const char *kb0 = reinterpret_cast<const char *>(Kh + (int64_t)key0 * nkt);
#pragma unroll
        for (int j = 0; j < LD; j++) {
            const int o = (wave * LD + j) * 1024 + lane * 16;
            const int r = o / RBYTES, pch = (o % RBYTES) / 16;
            tile_dma16(kb0, (uint32_t)(r * nkt * 4 + (pch ^ (r & (F - 1))) * 16), ks_base + j * 1024);
        }
    };
    auto dma_v = [&](int key0) {
        const char *vb0 = reinterpret_cast<const char *>(Vh + (int64_t)key0 * nkt);
#pragma unroll
        for (int j = 0; j < LD; j++) {
            const int o = (wave * LD + j) * 1024 + lane * 16;
            const int r = o / RBYTES, pch = (o % RBYTES) / 16;
            tile_dma16(vb0, (uint32_t)(r * nkt * 4 + pch * 16), vs_base + j * 1024);
        }
    };
    dma_k(kt0 * KT);
    dma_v(kt0 * KT);

    // Q fragment: dims [grp*DQ, grp*DQ + DQ) of query row (t, h), pre-multiplied by
    // scale * log2(e) so the S^T accumulators are already in base-2 units.
    float qf[DQ];
    {
        const float *qrow = p.q + ((int64_t)(tok_ok ? t : 0) * p.n_head + h) * p.hd + grp * DQ;
#pragma unroll
        for (int s = 0; s < DQ; s++) qf[s] = qrow[s] * p.qscale;
    }

    // Smallest and largest position among this wave's 16 tokens (invalid columns do not
    // count towards the minimum).
    int wmax = pq, wmin = tok_ok ? pq : 0x7fffffff;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        wmax = max(wmax, __shfl_xor(wmax, off));
        wmin = min(wmin, __shfl_xor(wmin, off));
    }

    floatx4 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; db++) oacc[db] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY, l = 0.0f;

    // Per tile: S and the softmax read K(t); a barrier; K(t+1)'s loads are issued (they
    // land while PV(t) runs); PV reads V(t); a barrier once this wave's K(t+1) has
    // landed; V(t+1)'s loads are issued (they land while S(t+1) runs) and waited for
    // before the next barrier.  The first tile's K and V were issued before the query.
    float sv[KB][4];
    for (int kt = kt0; kt < kt1; kt++) {
        const int key0 = kt * KT;
        // V rows past the largest position among the block's queries have weight 0 for
        // every query; they are set to zero, so that a non-finite value in a row no
        // window of the block contains cannot turn 0 * V into NaN.
        const bool tail = key0 + KT - 1 > kmax;
        // Tiles reaching past the smallest position hold keys some query must not weigh.
        const bool diag = key0 + KT - 1 > kmin;
        const bool active = head_ok && key0 <= wmax;
        if (kt == kt0) {
            wait_tile_dma();
            __syncthreads();
        }
        if (active) {
            // S^T = K Q^T for KB blocks of 16 keys; independent accumulators interleaved.
            floatx4 sacc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; kb++) sacc[kb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < DQ; s += 4) {
                float4 kf[KB];
#pragma unroll
                for (int kb = 0; kb < KB; kb++)
                    kf[kb] = *reinterpret_cast<const float4 *>(&Ks[(kb * 16 + qc) * KSTR + (((grp * DQ + s) / 4) ^ (qc & (F - 1))) * 4]);
#pragma unroll
                for (int kb = 0; kb < KB; kb++) sacc[kb] = mfma4(kf[kb].x, qf[s + 0], sacc[kb]);
#pragma unroll
                for (int kb = 0; kb < KB; kb++) sacc[kb] = mfma4(kf[kb].y, qf[s + 1], sacc[kb]);
#pragma unroll
                for (int kb = 0; kb < KB; kb++) sacc[kb] = mfma4(kf[kb].z, qf[s + 2], sacc[kb]);
#pragma unroll
                for (int kb = 0; kb < KB; kb++) sacc[kb] = mfma4(kf[kb].w, qf[s + 3], sacc[kb]);
            }
            // Mask keys beyond this query's position (only tiles that reach past the
            // wave's smallest position need the compare).
            float tmax = -INFINITY;
            if (key0 + KT - 1 <= wmin) {
#pragma unroll
                for (int kb = 0; kb < KB; kb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        sv[kb][r] = sacc[kb][r];
                        tmax = fmaxf(tmax, sv[kb][r]);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < KB; kb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int key = key0 + kb * 16 + grp * 4 + r;
                        sv[kb][r] = key <= pq ? sacc[kb][r] : -INFINITY;
                        tmax = fmaxf(tmax, sv[kb][r]);
                    }
            }
            tmax = max_xor32(max_xor16(tmax));
            // Key 0 is in tile 0 and every window holds it, so from tile 0 on mn is finite;
            // a segment that starts later can see a query none of whose keys it holds yet
            // (mn = -inf): mref = 0 then keeps its weights at exp2(-inf) = 0.
            const float mn = fmaxf(m, tmax);
            const float mref = mn == -INFINITY ? 0.0f : mn;
            // The running max moves rarely after the first tiles: rescale only when some
            // lane's did (alpha = 1 exactly otherwise).
            if (__any(mn != m)) {
                const float alpha = fast_exp2(m - mref);
                l *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; db++) oacc[db] *= alpha;
            }
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float pr = fast_exp2(sv[kb][r] - mref);
                    sv[kb][r] = pr;
                    l += pr;
                }
            m = mn;
        }
        wait_tile_dma();   // V(t) landed (issued last tile, or with K for the first)
        __syncthreads();   // K(t) read by every wave; V(t) landed everywhere
        if (kt + 1 < kt1) dma_k(key0 + KT);
        // In a tile past the smallest position a non-finite V value is set to 0 (its
        // neighbours unchanged) and the block is flagged: 0 * inf in the products would
        // turn the zero weight of a query whose window does not hold it into NaN; the
        // queries whose windows hold one add it at the end.  In the other tiles every
        // weight is positive and the products carry inf and NaN as they are.  This pass
        // reads and rewrites the tile in LDS (one more barrier), on such tiles only.
        if (tail || diag) {
            bool vbad = false;
#pragma unroll
            for (int j = 0; j < LD; j++) {
                const int idx = (tid + 256 * j) * 4;
                const int row = idx / HD;
                floatx4 v = *reinterpret_cast<const floatx4 *>(&Vs[idx]);
                bool chg = false;
                if (tail && key0 + row > kmax) {
                    v = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                    chg = true;
                } else if (diag) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const bool f = __builtin_isfinite(v[i]);
                        vbad |= !f;
                        chg |= !f;
                        v[i] = f ? v[i] : 0.0f;
                    }
                }
                if (chg) *reinterpret_cast<floatx4 *>(&Vs[idx]) = v;
            }
            if (vbad) s_vbad = 1;
            __syncthreads();
        }
        if (active) {
            // O^T += V^T P^T.  k-step st = 4 kb + r uses key kb*16 + 4*grp + r for lane
            // group grp.  Output block db = VEC*j + e takes, for A row i, dim
            // 16*VEC*j + VEC*i + e, so one VEC-wide LDS read (dims 16*VEC*j + VEC*qc ...)
            // feeds VEC blocks.  A step's V values are read while the previous step's
            // MFMAs run (the scheduling barriers keep that order: left alone, the compiler
            // puts each read just before its MFMAs and the wave waits on LDS every step).
            auto load_v = [&](int st, float (&vv)[NDB]) {
                const float *vrow = &Vs[((st >> 2) * 16 + grp * 4 + (st & 3)) * VSTR + VEC * qc];
#pragma unroll
                for (int j = 0; j < NDB / VEC; j++) {
                    if constexpr (VEC == 4) {
                        const float4 v4 = *reinterpret_cast<const float4 *>(vrow + 16 * VEC * j);
                        vv[4 * j] = v4.x; vv[4 * j + 1] = v4.y; vv[4 * j + 2] = v4.z; vv[4 * j + 3] = v4.w;
                    } else if constexpr (VEC == 2) {
                        const float2 v2 = *reinterpret_cast<const float2 *>(vrow + 16 * VEC * j);
                        vv[2 * j] = v2.x; vv[2 * j + 1] = v2.y;
                    } else {
                        vv[j] = vrow[16 * VEC * j];
                    }
                }
            };
            float vbuf[2][NDB];
            load_v(0, vbuf[0]);
#pragma unroll
            for (int st = 0; st < KB * 4; st++) {
                if (st + 1 < KB * 4) load_v(st + 1, vbuf[(st + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int db = 0; db < NDB; db++)
                    oacc[db] = mfma4(vbuf[st & 1][db], sv[st >> 2][st & 3], oacc[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_tile_dma();   // K(t+1) landed
        __syncthreads();   // V(t) read by every wave; K(t+1) landed everywhere
        if (kt + 1 < kt1) dma_v(key0 + KT);
    }

    // Non-finite V values inside this lane's window (keys of this unit's tiles up to its
    // position): the weighted sum is non-finite whatever their (positive) weights, and
    // adding the values themselves gives the same inf, -inf or NaN (adding again one that
    // the products already carried changes nothing).  The flag was set before the last
    // tile's barrier, so every wave reads the same value.
    if (s_vbad && head_ok && tok_ok) {
        const int kend = min(kt1 * KT, pq + 1);
        for (int key = kt0 * KT; key < kend; key++) {
            const KVT *vrow = Vh + (int64_t)key * nkt;
#pragma unroll
            for (int db = 0; db < NDB; db++)
#pragma unroll
                for (int rr = 0; rr < 4; rr++) {
                    const float v = (float)vrow[16 * VEC * (db / VEC) + VEC * (4 * grp + rr) + db % VEC];
                    if (!__builtin_isfinite(v)) oacc[db][rr] += v;
                }
        }
    }

    l = add_xor32(add_xor16(l));
    if (head_ok && tok_ok) {
        // Block VEC*j + e, register r' holds dim 16*VEC*j + VEC*(4*grp + r') + e: for each
        // (j, r') the VEC dims e = 0..VEC-1 are contiguous.  A split query tile writes
        // its segment's record instead of the output; the merge kernel reads a token's
        // segment count from segment 0's record.
        float inv = 1.0f / l;
        float *orow = p.out + ((int64_t)t * p.n_head + h) * HD;
        if (p.part) {
            float *rec = part_record<HD>(p, seg, t, h);
            if (grp == 0) {
                rec[HD] = m;
                rec[HD + 1] = l;
                if (seg == 0) rec[HD + 2] = __int_as_float(nseg);
            }
            if (nseg > 1) {
                orow = rec;
                inv = 1.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < NDB / VEC; j++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                float *dst = orow + 16 * VEC * j + VEC * (4 * grp + rr);
                if constexpr (VEC == 4) {
                    *reinterpret_cast<float4 *>(dst) =
                        make_float4(oacc[4 * j][rr] * inv, oacc[4 * j + 1][rr] * inv,
                                    oacc[4 * j + 2][rr] * inv, oacc[4 * j + 3][rr] * inv);
                } else if constexpr (VEC == 2) {
                    *reinterpret_cast<float2 *>(dst) =
                        make_float2(oacc[2 * j][rr] * inv, oacc[2 * j + 1][rr] * inv);
                } else {
                    dst[0] = oacc[j][rr] * inv;
                }
            }
    }
}

// Merge of the split query tiles' segment records: thread group of HD/4 lanes per
// (token, head), four dims per lane.  out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// folded online over batches of kBatch records whose loads are all in flight together
// (the first batch's alongside the segment count: records below max_seg exist, and those
// past the count are discarded by a select).
template <int HD>
__global__ void __launch_bounds__(256) prefill_merge_kernel(PrefillParams p)
{
    constexpr int TPR = HD / 4;           // threads per record
    constexpr int RPB = 256 / TPR;        // records per workgroup
    constexpr int kBatch = 8;
    if ((int)threadIdx.x >= RPB * TPR) return;   // head dims that do not divide 1,024
    const int rec = (int)blockIdx.x * RPB + (int)threadIdx.x / TPR;
    const int d = ((int)threadIdx.x % TPR) * 4;
    if (rec >= p.nt * p.n_head) return;
    const int t = rec / p.n_head, h = rec - t * p.n_head;
    const int nseg = __float_as_int(part_record<HD>(p, 0, t, h)[HD + 2]);
    float M = -INFINITY, L = 0.0f;
    floatx4 O = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < p.max_seg; s0 += kBatch) {
        float mi[kBatch], li[kBatch];
        floatx4 oi[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; i++) {
            const float *r = part_record<HD>(p, min(s0 + i, p.max_seg - 1), t, h);
            mi[i] = r[HD];
            li[i] = r[HD + 1];
            oi[i] = *reinterpret_cast<const floatx4 *>(r + d);
        }
        if (s0 == 0 && nseg <= 1) return;   // written by its only segment
        float Mn = M;
#pragma unroll
        for (int i = 0; i < kBatch; i++) {
            if (s0 + i >= nseg) mi[i] = -INFINITY;
            Mn = fmaxf(Mn, mi[i]);
        }
        // Segment 0 holds key 0, so Mn is finite from the first batch on.
        const float a = fast_exp2(M - Mn);
        L *= a;
        O *= a;
#pragma unroll
        for (int i = 0; i < kBatch; i++) {
            const bool live = s0 + i < nseg;   // 0 weight also for m = -inf (no key seen)
            const float w = live ? fast_exp2(mi[i] - Mn) : 0.0f;
            L += w * (live ? li[i] : 0.0f);
            O += w * (live ? oi[i] : floatx4{0.0f, 0.0f, 0.0f, 0.0f});
        }
        M = Mn;
        if (s0 + kBatch >= nseg) break;
    }
    const float inv = 1.0f / L;
    *reinterpret_cast<floatx4 *>(p.out + ((int64_t)t * p.n_head + h) * HD + d) = O * inv;
}

template <int HD, typename KVT>
hipError_t launch_hd_t(const PrefillParams &p, hipStream_t s)
{
    const int nblocks = p.units_per_hgroup * p.n_head_kv * p.n_hsub;
    const int launched = (nblocks + 7) / 8 * 8;
    prefill_kernel<HD, KVT><<<dim3((unsigned)launched), dim3(256), 0, s>>>(p, nblocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.part) return e;
    const int per_block = 256 / (HD / 4);
    const int64_t recs = (int64_t)p.nt * p.n_head;
    prefill_merge_kernel<HD><<<dim3((unsigned)((recs + per_block - 1) / per_block)), dim3(256), 0, s>>>(p);
    return hipGetLastError();
}

template <int HD>
hipError_t launch_hd(const PrefillParams &p, hipStream_t s)
{
    return launch_hd_t<HD, float>(p, s);
}

// binary16 regions: rows [0, dq_rows) of the window widened once into an f32 copy (each
// thread 4 consecutive values; blockIdx.y = 0 the K region, 1 the V region after it).
__global__ void __launch_bounds__(256) widen_f16_kernel(const _Float16 *kreg, const _Float16 *vreg,
                                                        int64_t n4, float *dst)
{
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n4) return;
    const _Float16 *src = blockIdx.y ? vreg : kreg;
    const half4_t h = reinterpret_cast<const half4_t *>(src)[g];
    reinterpret_cast<floatx4 *>(dst + blockIdx.y * n4 * 4)[g] =
        floatx4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

// Q8_0 regions: rows [0, dq_rows) of the window are dequantized once into an f32 copy
// with the region's row layout (value = scale * code, exact in f32), and the f32 kernel
// runs on the copy.  Dequantizing inside every workgroup's tile copy instead repeats it
// for each query tile of a kv head.  A workgroup converts 1024 groups of 4 values (one
// code word, one scale each), lane-contiguous in every load and store; blockIdx.y = 0
// reads the K region into dst[0, 4 * n4), 1 the V region after it.
__global__ void __launch_bounds__(256) dequant_q8_kernel(const char *kreg, const char *vreg,
                                                         int64_t scale_off, int32_t nkt,
                                                         int32_t hd_kv, int64_t n4, float *dst)
{
    const char *region = blockIdx.y ? vreg : kreg;
    dst += blockIdx.y * n4 * 4;
    const int64_t rows = scale_off / nkt;
    const _Float16 *sc = reinterpret_cast<const _Float16 *>(region + scale_off);
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const int64_t g = (int64_t)blockIdx.x * 1024 + w * 256 + threadIdx.x;
        if (g >= n4) return;
        const int64_t v0 = g * 4;
        const int64_t row = v0 / nkt;
        const int32_t c = *reinterpret_cast<const int32_t *>(region + v0);
        const float d = (float)sc[q8_scale_index(row, (int32_t)(v0 - row * nkt), hd_kv, rows)];
        reinterpret_cast<floatx4 *>(dst)[g] =
            floatx4{d * (float)(int8_t)c, d * (float)(int8_t)(c >> 8),
                    d * (float)(int8_t)(c >> 16), d * (float)(int8_t)(c >> 24)};
    }
}

hipError_t launch_by_hd(const PrefillParams &p, hipStream_t s)
{
    switch (p.hd_kv) {
    case 16: return launch_hd<16>(p, s);
    case 32: return launch_hd<32>(p, s);
    case 64: return launch_hd<64>(p, s);
    case 80: return launch_hd<80>(p, s);
    case 96: return launch_hd<96>(p, s);
    case 112: return launch_hd<112>(p, s);
    case 128: return launch_hd<128>(p, s);
    case 160: return launch_hd<160>(p, s);
    case 192: return launch_hd<192>(p, s);
    case 256: return launch_hd<256>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, hipStream_t s)
{
    if (p.nt <= 0) return hipSuccess;
    if (p.kv_fmt == kFmtF32) return launch_by_hd(p, s);
    if (!p.dq || p.dq_rows <= 0) return hipErrorInvalidValue;
    const int32_t nkt = p.n_head_kv * p.hd_kv;
    const int64_t vals = (int64_t)p.dq_rows * nkt;
    const int64_t n4 = vals / 4;
    PrefillParams f = p;
    f.kc = p.dq;
    f.vc = p.dq + vals;
    f.kv_fmt = kFmtF32;
    f.scale_off = 0;
    if (p.kv_fmt == kFmtQ8) {
        dequant_q8_kernel<<<dim3((unsigned)((n4 + 1023) / 1024), 2), dim3(256), 0, s>>>(
            static_cast<const char *>(p.kc), static_cast<const char *>(p.vc), p.scale_off, nkt,
            p.hd_kv, n4, p.dq);
    } else {
        widen_f16_kernel<<<dim3((unsigned)((n4 + 255) / 256), 2), dim3(256), 0, s>>>(
            static_cast<const _Float16 *>(p.kc), static_cast<const _Float16 *>(p.vc), n4, p.dq);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_by_hd(f, s);
}

}  // namespace kvc
