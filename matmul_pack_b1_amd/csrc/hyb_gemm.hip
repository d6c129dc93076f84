// Matrix-core kernels of libhyb (gfx950): the register-fed GEMM for up to
// about 128 tokens and the LDS-staged GEMM above, both with sparse tiles on
// the sparse matrix instructions, plus the host routing between them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "hyb_device.h"

namespace hyb {
namespace {

// ---------------------------------------------------------------- GEMM ----
//
// Y[m, n] = sum_k X[m, k] W'[n, k] for any M on the matrix cores
// (k_gemm_rx up to 128 tokens, k_gemm_lds above).  A K step is 64 columns
// and a wavefront's unit is 64 weight rows (four 16-row slabs).  A sparse
// slab piece is one v_smfmac_*_16x16x64 A operand (32 kept values per row)
// with its 2-bit indices: the stored value chunk and its idx2 word are
// exactly that instruction's operand layout, so sparse tiles run on the
// sparse matrix cores with no expansion.  Both kinds take the same B
// operands (X[m][8q..8q+7] and X[m][32+8q..32+8q+7] for lane group q).
// Partial sums are always added in a fixed order, so results are
// reproducible.
// Adds the low-rank term sum_j U[row][j] T[tok][j] (3BASiL, gist.science,
// section 1: W ~ S + L with L = U V^T, and T = X V) to a block of 16 x 16
// accumulator tiles: slab s holds rows row0 + 16 s, token block b tokens
// tok0 + 16 b (lane L: rows 4 (L/16) + 0..3 of the slab, token L%16), the
// layout of the products above.  Per 32-wide slice of the rank each slab's
// U piece and each token block's T piece is loaded once.  With bf16
// weights T is split into bf16 hi + lo (|T - hi - lo| <= 2^-16 |T|) and
// each tile takes two exact 16x16x32 products; with fp16 weights (where a
// 16-bit T could overflow) the fp32 16x16x4 instruction takes the products,
// lane group q supplying j = j0 + 8q + e to step e of both operands.  Rows
// are whole (n is a multiple of 64); tokens >= m and j >= rank read as zero.
template <int DT, int NS, int NT>
__device__ __forceinline__ void lr_block(f32x4_t (&c)[NS][NT], const GemmDims& d, int64_t row0, int64_t tok0,
                                         int lane) {
  const int q = lane >> 4, r = lane & 15;
  for (int32_t j0 = 0; j0 < d.rank; j0 += 32) {
    const int32_t j = j0 + 8 * q;
    const bool j_ok = j < d.rank;
    uint4 uw[NS];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
      uw[sl] = j_ok ? *reinterpret_cast<const uint4*>(d.u + (row0 + 16 * sl + r) * d.ldu + j)
                    : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int64_t tok = tok0 + 16 * b + r;
      float4 t0 = make_float4(0.f, 0.f, 0.f, 0.f), t1 = t0;
      if (j_ok && tok < d.m) {
        t0 = *reinterpret_cast<const float4*>(d.t + tok * d.ldt + j);
        t1 = *reinterpret_cast<const float4*>(d.t + tok * d.ldt + j + 4);
      }
      const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
      if constexpr (DT == HYB_BF16) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h0 = round16<HYB_BF16>(tv[2 * e]), h1 = round16<HYB_BF16>(tv[2 * e + 1]);
          const uint32_t l0 = round16<HYB_BF16>(tv[2 * e] - widen16<HYB_BF16>(h0));
          const uint32_t l1 = round16<HYB_BF16>(tv[2 * e + 1] - widen16<HYB_BF16>(h1));
          hi[e] = h0 | (h1 << 16);
          lo[e] = l0 | (l1 << 16);
        }
        const uint4 bh = make_uint4(hi[0], hi[1], hi[2], hi[3]), bl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          c[sl][b] = mfma16x16x32<HYB_BF16>(uw[sl], bh, c[sl][b]);
          c[sl][b] = mfma16x16x32<HYB_BF16>(uw[sl], bl, c[sl][b]);
        }
      } else {
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          const uint32_t w4[4] = {uw[sl].x, uw[sl].y, uw[sl].z, uw[sl].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            c[sl][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(widen16<DT>(e & 1 ? w4[e >> 1] >> 16 : w4[e >> 1] & 0xFFFFu),
                                                            tv[e], c[sl][b], 0, 0, 0);
        }
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ f32x4_t smfmac16x16x64(uint4 a, uint4 b0, uint4 b1, uint32_t idx, f32x4_t c) {
  const uint32_t bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  if constexpr (DT == HYB_BF16) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                     __builtin_bit_cast(bf16x16_t, bb), c, idx, 0, 0);
  } else {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(half8_t, a),
                                                    __builtin_bit_cast(half16_t, bb), c, idx, 0, 0);
  }
}

// 2-bit index word (i0 | i1 << 2 per group) from a metadata word.
template <int META>
__device__ __forceinline__ uint32_t idx2_word(uint32_t word) {
  if constexpr (META == HYB_META_MASK8) {
    return 0u;  // 4:8 groups have no 2-bit index word; their paths never ask
  } else if constexpr (META == HYB_META_IDX2) {
    return word & 0xFFFFu;
  } else {
    uint32_t out = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t i0, i1;
      nibble_positions_t<HYB_META_MASK4>((word >> (4 * g)) & 0xFu, i0, i1);
      out |= ((i0 & 3u) | ((i1 & 3u) << 2)) << (4 * g);
    }
    return out;
  }
}

// --------------------------------------------------- GEMM (register-fed) --
//
// Memory-bound range (17 to a few hundred tokens): the weights must stream
// at the decode kernel's rate while the tokens are multiplied on the matrix
// cores.  A workgroup owns 64 weight rows (four 16-row slabs) and BM = 16*MB
// tokens; its WAVES wavefronts split the K steps into contiguous ranges, as
// the decode kernel's do, and never synchronise inside the K walk.  Each
// lane loads exactly its operands straight into a STAGES-deep register
// ring: its slab pieces and, from L2, its B operands
// X[m][8q..8q+7] and X[m][32+8q..32+8q+7] of every token block.  Past the
// end of a wavefront's range, or past the last token row, the loads fall
// outside the buffer resources and read zero, so every trip issues the same
// loads.  At the end the wavefronts' partial sums are added through LDS in
// a fixed tree order (reproducible results).
// One step's operands for one lane: per slab two 16-byte weight pieces (the
// two halves of a dense piece's 2:4 split, or the sparse chunk and zeros)
// and the aligned dword holding the sparse metadata word (a 16-bit load is
// zero-extended by the compiler where it lands, which waits for it and
// drains the ring); the B operands of every token block; the tile index.
template <int MB, int RG>
struct GemmRxStage {
  u32x4_t v0[RG][4], v1[RG][4];
  uint32_t m[RG][4];
  uint4 b[MB][2];
  int32_t ti[RG];
};

// One piece of a register-fed product: K steps [k0, k1) of the tile of
// 64*RG weight rows from n0 and BM = 16*MB tokens from m0.  The WAVES
// wavefronts split the piece's K steps into contiguous ranges and never
// synchronise inside the K walk; their sums are then added through LDS
// (WAVES/2 wavefront-sized buffers) in a fixed tree order, so that
// wavefront 0 ends with the piece's sum in `acc` (the other wavefronts'
// `acc` are left partial).  The piece that starts at K step 0 also adds the
// low-rank term.  The LDS arrays are declared here rather than passed in so
// that every access to them is a known LDS access.
template <int B2, int DT, int META, int MB, int WAVES, int STAGES, int RG>
__device__ __forceinline__ void rx_piece(const uint4* __restrict__ dense, const uint4* __restrict__ val,
                                         const uint16_t* __restrict__ meta, const int32_t* __restrict__ tidx,
                                         const uint16_t* __restrict__ x, const GemmDims& d, int32_t n0,
                                         int32_t m0, int32_t k0, int32_t k1, f32x4_t (&acc_out)[RG][4][MB]) {
  f32x4_t acc[RG][4][MB];
  static_assert(WAVES == 4 || WAVES == 8, "tree reduction over 4 or 8 wavefronts");
  constexpr int BM = 16 * MB;
  constexpr int kStepsPerTile = B2 / 64;
  constexpr int kPart = RG * 4 * MB * 64 * 4;  // floats of one wavefront's partial sums
  __shared__ __attribute__((aligned(16))) float red[WAVES / 2][kPart];
  __shared__ uint4 lut8[META == HYB_META_MASK8 ? 256 : 1];
  if constexpr (META == HYB_META_MASK8) {
    fill_expand8_lut(lut8);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int r = lane & 15;
  const int32_t steps = k1 - k0;
  const int32_t s0 = k0 + (wave * steps) / WAVES;
  const int32_t cnt = k0 + ((wave + 1) * steps) / WAVES - s0;
  const int32_t mrows = d.m - m0 < BM ? d.m - m0 : BM;
  const int64_t tile = int64_t(d.b1) * B2;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + int64_t(m0) * d.ldx, mrows * int32_t(d.ldx) * 2);
  // Lane L's 2:4 operand of a dense slab covers columns 16q..16q+15 of the
  // step: lane groups 2(q%2) and 2(q%2)+1 of dense chunk q/2.
  const int dense_off = (q >> 1) * 1024 + ((2 * (q & 1)) * 16 + r) * 16;

  constexpr int32_t kNone = INT32_MIN;
  auto load = [&](GemmRxStage<MB, RG>& st, int32_t it) {
    const bool live = it < cnt;
    const int kb = (s0 + it) % kStepsPerTile;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int32_t ng = n0 + 64 * g;
      const bool rows = ng < d.n;
      const int32_t tn = rows ? ng / d.b1 : 0;
      const int rs0 = (ng - tn * d.b1) / 16;
      int32_t ti = (live && rows) ? tidx[int64_t(tn) * d.tiles_k + (s0 + it) / kStepsPerTile] : kNone;
      const bool is_dense = ti >= 0;
      const int32_t slot = is_dense ? ti : ~ti;
      if (is_dense ? (slot >= d.n_dense) : (slot >= d.n_sparse)) ti = kNone;
      st.ti[g] = ti;
      const bool ok = ti != kNone;
      const int32_t slab_bytes = is_dense ? 32 * B2 : 16 * B2;
      const char* base = is_dense
          ? reinterpret_cast<const char*>(dense) + (int64_t(slot) * tile + int64_t(rs0) * 16 * B2) * 2
          : reinterpret_cast<const char*>(val) + (int64_t(slot) * (tile / 2) + int64_t(rs0) * 8 * B2) * 2;
      const __amdgpu_buffer_rsrc_t ar = make_rsrc(ok ? base : nullptr, ok ? 4 * slab_bytes : 0);
      const char* mbase = reinterpret_cast<const char*>(meta) + (int64_t(slot) * (tile / 16) + int64_t(rs0) * B2) * 2;
      const __amdgpu_buffer_rsrc_t mr =
          make_rsrc((ok && !is_dense) ? mbase : nullptr, (ok && !is_dense) ? 8 * B2 : 0);
      const int32_t o0 = is_dense ? 2 * kb * 1024 + dense_off : kb * 1024 + lane * 16;
      const int32_t o1 = is_dense ? o0 + 256 : 0x40000000;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        st.v0[g][sl] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, sl * slab_bytes + o0, 0, 0));
        st.v1[g][sl] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, sl * slab_bytes + o1, 0, 0));
        st.m[g][sl] = __builtin_amdgcn_raw_buffer_load_b32(mr, (sl * 2 * B2 + lane * (B2 / 32) + kb * 2) & ~3, 0, 0);
      }
    }
    const int32_t col = live ? (s0 + it) * 128 + q * 16 : 0x40000000;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int32_t row = (mb * 16 + r) * int32_t(d.ldx) * 2;
      st.b[mb][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, row + col, 0, 0));
      st.b[mb][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, row + col + 64, 0, 0));
    }
  };

#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j) acc[g][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Every slab runs on v_smfmac: the first pass for both kinds (a sparse
  // chunk with its index word, or positions 0,1 of every group of a dense
  // piece, index 0x4444), the second pass for dense slabs (positions 2,3,
  // index 0xEEEE).  The selects are bit-selects on an opaque mask so they
  // stay branch-free.
  auto compute = [&](const GemmRxStage<MB, RG>& st, int32_t it) {
    const int mshift = ((lane * (B2 / 32) + ((s0 + it) % kStepsPerTile) * 2) & 2) * 8;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const int32_t ti = st.ti[g];
      if (ti == kNone) continue;
      const bool is_dense = ti >= 0;
      uint32_t dm = is_dense ? ~0u : 0u;
      asm("" : "+v"(dm));
      uint4 a0[4], a1[4];
      uint32_t i0[4];
      if constexpr (META == HYB_META_MASK8) {
        // 4:8: a sparse slab's sixteen columns per lane, expanded, take the
        // place of the dense slab's two chunk pieces; both kinds run both
        // passes.
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const u32x4_t v0 = st.v0[g][sl], v1 = st.v1[g][sl];
          uint32_t e[8];
          expand8_lane(lut8, v0[0], v0[1], v0[2], v0[3], (st.m[g][sl] >> mshift) & 0xFFFFu, e);
          const uint32_t l0 = bitsel(dm, v0[0], e[0]), l1 = bitsel(dm, v0[1], e[1]);
          const uint32_t l2 = bitsel(dm, v0[2], e[2]), l3 = bitsel(dm, v0[3], e[3]);
          const uint32_t h0 = bitsel(dm, v1[0], e[4]), h1 = bitsel(dm, v1[1], e[5]);
          const uint32_t h2 = bitsel(dm, v1[2], e[6]), h3 = bitsel(dm, v1[3], e[7]);
          a0[sl] = make_uint4(l0, l2, h0, h2);
          a1[sl] = make_uint4(l1, l3, h1, h3);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            acc[g][sl][mb] = smfmac16x16x64<DT>(a0[sl], st.b[mb][0], st.b[mb][1], 0x4444u, acc[g][sl][mb]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            acc[g][sl][mb] = smfmac16x16x64<DT>(a1[sl], st.b[mb][0], st.b[mb][1], 0xEEEEu, acc[g][sl][mb]);
        continue;
      }
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const u32x4_t v0 = st.v0[g][sl], v1 = st.v1[g][sl];
        a0[sl] = make_uint4(v0[0], bitsel(dm, v0[2], v0[1]), bitsel(dm, v1[0], v0[2]), bitsel(dm, v1[2], v0[3]));
        u32x4_t t = {v0[1], v0[3], v1[1], v1[3]};
        asm("" : "+v"(t));
        a1[sl] = __builtin_bit_cast(uint4, t);
        i0[sl] = bitsel(dm, 0x4444u, idx2_word<META>((st.m[g][sl] >> mshift) & 0xFFFFu));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[g][sl][mb] = smfmac16x16x64<DT>(a0[sl], st.b[mb][0], st.b[mb][1], i0[sl], acc[g][sl][mb]);
      if (is_dense) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            acc[g][sl][mb] = smfmac16x16x64<DT>(a1[sl], st.b[mb][0], st.b[mb][1], 0xEEEEu, acc[g][sl][mb]);
      }
    }
  };

  // STAGES-deep ring, unrolled so every stage index is a compile-time
  // constant; loads of the next STAGES-1 steps are in flight while a step
  // is multiplied.
  GemmRxStage<MB, RG> st[STAGES];
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) load(st[s], s);
  for (int32_t i = 0; i < cnt; i += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      load(st[(s + STAGES - 1) % STAGES], i + s + STAGES - 1);
      if (i + s < cnt) compute(st[s], i + s);
    }
  }

  // Low-rank term: token block mb by wavefront mb % WAVES, into that
  // wavefront's partial sums (the tree below keeps a fixed order).
  if (d.rank > 0 && k0 == 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb % WAVES != wave) continue;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        if (n0 + 64 * g >= d.n) continue;
        f32x4_t c[4][1] = {{acc[g][0][mb]}, {acc[g][1][mb]}, {acc[g][2][mb]}, {acc[g][3][mb]}};
        lr_block<DT, 4, 1>(c, d, n0 + 64 * g, m0 + 16 * mb, lane);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) acc[g][sl][mb] = c[sl][0];
      }
    }
  }

  // Tree reduction: wavefronts w >= h hand their sums to w - h, for
  // h = WAVES/2, ..., 1.  The closing barrier also keeps `red` free for the
  // next piece.
#pragma unroll
  for (int h = WAVES / 2; h >= 1; h /= 2) {
    if (wave >= h && wave < 2 * h) {
      float* dst = red[wave - h];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            *reinterpret_cast<f32x4_t*>(dst + (((g * 4 + sl) * MB + mb) * 64 + lane) * 4) = acc[g][sl][mb];
    }
    __syncthreads();
    if (wave < h) {
      const float* src = red[wave];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[g][sl][mb] += *reinterpret_cast<const f32x4_t*>(src + (((g * 4 + sl) * MB + mb) * 64 + lane) * 4);
    }
    __syncthreads();
  }
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc_out[g][sl][mb] = acc[g][sl][mb];
}

// Four outputs y[m][n..n+3] (fp32, or rounded to bf16 / fp16).
__device__ __forceinline__ void store_row4(void* y, const GemmDims& d, int64_t m, int64_t n, f32x4_t v,
                                           bool vec_ok) {
  const int64_t base = m * d.ldy + n;
  if (d.ydt == HYB_F32) {
    float* dst = static_cast<float*>(y) + base;
    if (vec_ok) {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = v[e];
    }
  } else {
    uint16_t* dst = static_cast<uint16_t*>(y) + base;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = d.ydt == HYB_BF16 ? round16<HYB_BF16>(v[e]) : round16<HYB_F16>(v[e]);
  }
}

__device__ __forceinline__ bool y_vec_ok(const void* y, const GemmDims& d) {
  return (d.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 15) == 0);
}

// acc[g][sl][mb] lane L holds rows n0 + 64 g + 16 sl + 4 (L/16) + 0..3 of
// token m0 + 16 mb + L%16.
template <int MB, int RG>
__device__ __forceinline__ void rx_store(const f32x4_t (&acc)[RG][4][MB], void* y, const GemmDims& d, int32_t n0,
                                         int32_t m0, int lane) {
  const bool vec_ok = y_vec_ok(y, d);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = int64_t(m0) + mb * 16 + (lane & 15);
    if (m >= d.m) continue;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      if (n0 + 64 * g >= d.n) continue;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        store_row4(y, d, m, int64_t(n0) + 64 * g + sl * 16 + (lane >> 4) * 4, acc[g][sl][mb], vec_ok);
    }
  }
}

// With four wavefronts and up to 64 tokens the launch bound asks for two
// wavefronts per SIMD (at most 256 registers each), so that two workgroups
// share a CU; 128 tokens, or two row groups per wavefront, need the whole
// register file of a SIMD.  RG is the number of 64-row groups per
// workgroup (each wavefront multiplies all of them over its K range: two
// groups halve the X reads per weight byte).
template <int MB, int WAVES, int RG>
constexpr int rx_occupancy() {
  return (WAVES == 4 && MB <= 4 && RG == 1) ? 2 : 1;
}

template <int B2, int DT, int META, int MB, int WAVES, int STAGES, int RG>
__global__ __launch_bounds__(64 * WAVES, (rx_occupancy<MB, WAVES, RG>())) void k_gemm_rx(
    const uint4* __restrict__ dense, const uint4* __restrict__ val, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ tidx, const uint16_t* __restrict__ x, void* __restrict__ y, GemmDims d) {
  const int32_t n0 = int32_t(blockIdx.x) * 64 * RG;
  const int32_t m0 = int32_t(blockIdx.y) * 16 * MB;
  f32x4_t acc[RG][4][MB];
  rx_piece<B2, DT, META, MB, WAVES, STAGES, RG>(dense, val, meta, tidx, x, d, n0, m0, 0,
                                                d.tiles_k * (B2 / 64), acc);
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) rx_store<MB, RG>(acc, y, d, n0, m0, threadIdx.x & 63);
}

// ------------------------------------------- GEMM (register-fed, split K) --
//
// When the tiles of a register-fed shape fill the compute units poorly
// (e.g. 136 tiles of 128 rows x 64 tokens on 256 CUs), the (row block, K
// step) units are dealt out evenly instead (the stream-K schedule).  Every
// token block gets the same G' workgroups' worth of split: unit
// u = nb * S + k (S K steps per tile) of token block mb, and of the G'
// ranges the first U mod G' hold floor(U / G') + 1 consecutive units, the
// rest floor(U / G') (U = row blocks * S).  Workgroup w = j * gm + mb runs
// range j of token block mb, so the gm workgroups that read the same weight
// rows at the same K steps are neighbours in launch order.  A workgroup's
// range covers whole tiles, stored directly, and at most two partial
// pieces: the piece its range starts in (workspace slot 2w) and the one it
// ends in (slot 2w + 1).  A second kernel then adds the pieces of every
// split tile in range order, a fixed order, so results are reproducible on
// a given device.
struct SplitPlan {
  int32_t units;   // U = row blocks * steps (< 2^31)
  int32_t steps;   // S, K steps per tile
  int32_t groups;  // G', ranges per token block (1 <= G' <= U)
  int32_t gm;      // token blocks
  int32_t q, r;    // U = q G' + r
};

constexpr int32_t kSplitXcds = 8;

// Launch arguments of a split product (groups 0: unsplit).
struct SplitArgs {
  int32_t groups;
  float* ws;
  int32_t rows0;  // GemmRoute::rows0
};

__device__ __forceinline__ int32_t split_begin(int32_t j, const SplitPlan& p) {
  return j * p.q + (j < p.r ? j : p.r);
}

// The range that holds unit u.
__device__ __forceinline__ int32_t split_owner(int32_t u, const SplitPlan& p) {
  const int32_t big = p.r * (p.q + 1);
  return u < big ? u / (p.q + 1) : p.r + (u - big) / p.q;
}

template <int B2, int DT, int META, int MB, int WAVES, int STAGES, int RG>
__global__ __launch_bounds__(64 * WAVES, (rx_occupancy<MB, WAVES, RG>())) void k_gemm_split(
    const uint4* __restrict__ dense, const uint4* __restrict__ val, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ tidx, const uint16_t* __restrict__ x, void* __restrict__ y, GemmDims d,
    SplitPlan p, float* __restrict__ ws) {
  constexpr int kPart = RG * 4 * MB * 64 * 4;
  const int lane = threadIdx.x & 63;
  const bool lead = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  // XCD-major order: launch slot L runs on XCD L % 8, and the workgroups of
  // one XCD take consecutive w, so neighbours in w share that XCD's L2.
  const int32_t G = int32_t(gridDim.x), L = int32_t(blockIdx.x);
  const int32_t xcd = L % kSplitXcds, per = G / kSplitXcds, extra = G % kSplitXcds;
  const int32_t w = xcd * per + (xcd < extra ? xcd : extra) + L / kSplitXcds;
  const int32_t j = w / p.gm, mb = w - j * p.gm;
  const int32_t m0 = mb * 16 * MB;
  const int32_t u1 = split_begin(j + 1, p);
  int slot = 0;
  for (int32_t u = split_begin(j, p); u < u1; ++slot) {
    const int32_t nb = u / p.steps;
    const int32_t ts = nb * p.steps;
    const int32_t k0 = u - ts;
    const int32_t k1 = (u1 < ts + p.steps ? u1 : ts + p.steps) - ts;
    const int32_t n0 = nb * 64 * RG;
    f32x4_t acc[RG][4][MB];
    rx_piece<B2, DT, META, MB, WAVES, STAGES, RG>(dense, val, meta, tidx, x, d, n0, m0, k0, k1, acc);
    if (lead) {
      if (k0 == 0 && k1 == p.steps) {
        rx_store<MB, RG>(acc, y, d, n0, m0, lane);
      } else {
        float* part = ws + (2 * int64_t(w) + (slot == 0 ? 0 : 1)) * kPart;
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
#pragma unroll
            for (int b = 0; b < MB; ++b)
              *reinterpret_cast<f32x4_t*>(part + (((g * 4 + sl) * MB + b) * 64 + lane) * 4) = acc[g][sl][b];
      }
    }
    u = ts + k1;
  }
}

// Adds the pieces of every split tile in workgroup order (the first
// owner's piece is its end piece unless its range starts at the tile, every
// later owner's is its start piece) and stores the sums.  One thread per
// four outputs (one float4 of a piece): kBlocks workgroups of 256 threads
// per tile; the workgroups of unsplit tiles return at once.
template <int MB, int RG>
__global__ __launch_bounds__(256) void k_gemm_split_sum(const float* __restrict__ ws, void* __restrict__ y,
                                                        GemmDims d, SplitPlan p) {
  constexpr int kVec = RG * 4 * MB * 64;  // float4 per piece
  constexpr int kBlocks = kVec / 256;
  const int32_t t = int32_t(blockIdx.x) / kBlocks;  // tile (row block t / gm, token block t % gm)
  const int32_t nb = t / p.gm, mt = t - nb * p.gm;
  const int32_t ts = nb * p.steps;
  const int32_t ja = split_owner(ts, p), jb = split_owner(ts + p.steps - 1, p);
  if (ja == jb) return;
  const int f = (int(blockIdx.x) % kBlocks) * 256 + int(threadIdx.x);
  const int64_t first = 2 * (int64_t(ja) * p.gm + mt) + (split_begin(ja, p) >= ts ? 0 : 1);
  f32x4_t s = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(ws + (first * kVec + f) * 4));
  for (int32_t j = ja + 1; j <= jb; ++j)
    s += __builtin_nontemporal_load(
        reinterpret_cast<const f32x4_t*>(ws + (2 * (int64_t(j) * p.gm + mt) * kVec + f) * 4));
  const int lane = f & 63;
  const int mb = (f >> 6) % MB;
  const int sl = ((f >> 6) / MB) & 3;
  const int g = (f >> 6) / (4 * MB);
  const int32_t n0 = nb * 64 * RG;
  const int64_t m = int64_t(mt) * 16 * MB + mb * 16 + (lane & 15);
  if (m >= d.m || n0 + 64 * g >= d.n) return;
  store_row4(y, d, m, int64_t(n0) + 64 * g + sl * 16 + (lane >> 4) * 4, s, y_vec_ok(y, d));
}

// ------------------------------------------------------------ GEMM (LDS) --
//
// Large-M variant: a workgroup covers 256 weight rows (four 64-row groups)
// and BM = 16 * MB tokens.  With four wavefronts each owns a row group and
// all BM tokens; with eight, two wavefronts share a row group and split the
// tokens.  Every K step (64 columns) the workgroup streams its weight pieces
// (8 x 1 KiB per row group: two chunks per slab, the second an empty
// out-of-range read for a sparse slab), the slabs' metadata words and the X
// tile (BM rows x 128 B) straight into LDS with buffer-load-to-LDS
// instructions, STAGES - 1 steps ahead, so the pipeline depth costs no
// registers.  The loads are issued from inline assembly: the compiler then
// does not tie every LDS read to every DMA in flight (which would drain the
// pipeline each step), and the waits are explicit -- every wavefront issues
// the same number of loads per step, so "at most (STAGES-2) steps of loads
// outstanding" followed by a workgroup barrier marks a step's LDS data
// complete and visible.  The X tile's 16-byte slots are XOR-swizzled by
// (row >> 1) & 7 so the B-operand reads of 16 rows hit distinct banks.
typedef __attribute__((ext_vector_type(4))) int srd_t;

__device__ __forceinline__ srd_t make_srd(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return srd_t{__builtin_amdgcn_readfirstlane(int(a & 0xFFFFFFFFu)),
               __builtin_amdgcn_readfirstlane(int((a >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane(int(bytes)), kBufDword3};
}

// 16 bytes per lane from srd + voffset into LDS at lds + 16 * lane.
template <bool NT>
__device__ __forceinline__ void dma16(srd_t srd, uint32_t lds, int voffset) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(lds), "v"(voffset), "s"(srd) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voffset), "s"(srd) : "memory", "m0");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  // generic -> LDS address space, then the 32-bit LDS offset
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Workgroups are dispatched round-robin over the 8 XCDs (linear id L runs
// on XCD L % 8), each XCD with its own L2.  The launch is a 1-D grid; XCD x
// takes a contiguous range of a grouped order in which kGroupN consecutive
// row blocks are swept across all token blocks before the next group, so the
// workgroups that run together on one XCD share both their weight rows and
// their X tiles in that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupN = HYB_GEMM_GROUP_N;

__device__ __forceinline__ void xcd_grouped_block(int32_t gx, int32_t& nb, int32_t& mb) {
  const int32_t total = int32_t(gridDim.x);  // gx row blocks x gy token blocks
  const int32_t gy = total / gx;
  const int32_t L = int32_t(blockIdx.x);
  const int32_t xcd = L % kXcds, j = L / kXcds;
  const int32_t per = total / kXcds, extra = total % kXcds;
  const int32_t g = xcd * per + (xcd < extra ? xcd : extra) + j;
  const int32_t gn = g / (kGroupN * gy);
  const int32_t first = gn * kGroupN;
  const int32_t width = gx - first < kGroupN ? gx - first : kGroupN;
  const int32_t r = g - first * gy;
  mb = r / width;
  nb = first + r % width;
}

// WAVES = 4: wavefront w owns rows 64w..64w+63 and all BM tokens.
// WAVES = 8: wavefronts w and w+4 share rows 64(w%4).. and split the tokens,
// giving two wavefronts per SIMD so one can multiply while the other waits
// at the barrier or on LDS.  Loads are spread so every wavefront issues the
// same number per step.
template <int B2, int MB, int STAGES, int WAVES>
struct GemmLdsCfg {
  static constexpr int kABytes = 4 * 8 * 1024;               // weight pieces of 4 row groups
  static constexpr int kXBytes = 16 * MB * 128;               // X tile
  static constexpr int kMetaPerGroup = B2 * 8 < 1024 ? 1024 : B2 * 8;
  static constexpr int kMetaBytes = 4 * kMetaPerGroup;
  static constexpr int kStage = kABytes + kXBytes + kMetaBytes;
  // An out-of-range DMA still writes (zeros) to LDS: loads issued only to
  // keep the per-step count constant land in this sink, which nothing reads.
  static constexpr int kSink = 1024;
  static constexpr int kBytes = STAGES * kStage + kSink;
  static constexpr int kSplit = WAVES / 4;                    // wavefronts per row group
  static constexpr int kALoads = 8 / kSplit;                  // weight chunks per wavefront
  static constexpr int kXLoads = kXBytes / 1024 / WAVES;      // X pieces per wavefront
  static constexpr int kMetaLoads = (kMetaPerGroup / 1024 + kSplit - 1) / kSplit;
  static constexpr int kLoadsPerStep = kALoads + kXLoads + kMetaLoads;
  static constexpr int kMBW = MB / kSplit;                    // token blocks per wavefront
};

// K steps [k0, k1) of the 256-row block nb and token block mbk: each
// wavefront ends with the sums of its own outputs in acc_out (wavefront w:
// row group w % 4, token half w / 4); no wavefront shares an output, so no
// reduction follows.  The closing barrier frees the LDS stages for the next
// piece.
template <int B2, int DT, int META, int MB, int STAGES, int WAVES>
__device__ __forceinline__ void lds_piece(const uint4* __restrict__ dense, const uint4* __restrict__ val,
                                          const uint16_t* __restrict__ meta, const int32_t* __restrict__ tidx,
                                          const uint16_t* __restrict__ x, const GemmDims& d, int32_t nb,
                                          int32_t mbk, int32_t k0, int32_t k1,
                                          f32x4_t (&acc_out)[4][GemmLdsCfg<B2, MB, STAGES, WAVES>::kMBW]) {
  using Cfg = GemmLdsCfg<B2, MB, STAGES, WAVES>;
  static_assert(Cfg::kXLoads >= 1 && Cfg::kXLoads * WAVES * 1024 == Cfg::kXBytes, "X tile split");
  constexpr int MBW = Cfg::kMBW;
  constexpr int BM = 16 * MB;
  constexpr int kStepsPerTile = B2 / 64;
  extern __shared__ __attribute__((aligned(1024))) char smem_dyn[];
  __shared__ uint4 lut8[META == HYB_META_MASK8 ? 256 : 1];
  // (4:8 only; the first barrier of the main loop precedes every read)
  if constexpr (META == HYB_META_MASK8) fill_expand8_lut(lut8);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % 4;            // row group
  const int wm = wave / 4;            // token half (WAVES = 8)
  const int q = lane >> 4;
  const int32_t n0 = nb * 256 + wn * 64;
  const int32_t m0 = mbk * BM;
  const bool rows_ok = n0 < d.n;
  const int32_t tn = n0 / d.b1;
  const int rs0 = (n0 - tn * d.b1) / 16;
  const int32_t* __restrict__ trow = tidx + int64_t(tn) * d.tiles_k;
  const int32_t mrows = d.m - m0 < BM ? d.m - m0 : BM;
  const int64_t tile = int64_t(d.b1) * B2;
  const uint32_t smem_base = lds_addr(smem_dyn);

  constexpr int32_t kNone = INT32_MIN;
  auto tile_index = [&](int32_t st) -> int32_t {
    if (!rows_ok || st >= k1) return kNone;
    const int32_t ti = trow[st / kStepsPerTile];
    const bool ok = ti >= 0 ? (ti < d.n_dense) : (~ti < d.n_sparse);
    return ok ? ti : kNone;
  };
  int32_t tis[STAGES];

  // Issue every load of step `st` into stage `sg` (a compile-time index).
  auto issue = [&](int32_t st, int sg, int32_t ti) {
    const uint32_t stage = smem_base + sg * Cfg::kStage;
    const int kb = st % kStepsPerTile;
    const bool live = ti != kNone;
    const bool is_dense = ti >= 0;
    const int32_t slot = is_dense ? ti : ~ti;
    const int32_t slab_bytes = is_dense ? 32 * B2 : 16 * B2;
    const char* base = is_dense
        ? reinterpret_cast<const char*>(dense) + (int64_t(slot) * tile + int64_t(rs0) * 16 * B2) * 2
        : reinterpret_cast<const char*>(val) + (int64_t(slot) * (tile / 2) + int64_t(rs0) * 8 * B2) * 2;
    const srd_t ar = make_srd(live ? base : nullptr, live ? 4 * slab_bytes : 0);
    const int32_t c0 = is_dense ? 2 * kb * 1024 : kb * 1024;
    const int32_t c1 = is_dense ? c0 + 1024 : 0x40000000;
    const uint32_t adst = stage + wn * 8192;
#pragma unroll
    for (int i = 0; i < Cfg::kALoads; ++i) {
      const int c = wm * Cfg::kALoads + i;   // chunk 2*sl + h of this row group
      const int sl = c >> 1;
      const int32_t off = (c & 1) ? c1 : c0;
      dma16<HYB_GEMM_W_NT != 0>(ar, adst + c * 1024, sl * slab_bytes + off + lane * 16);
    }
    // X tile: piece j (8 rows x 128 B); wavefront w loads pieces
    // w * kXLoads ..; lane l -> row 8j + l/8, LDS slot l%8 holding global
    // 16-byte column (l%8) ^ ((row >> 1) & 7).
    const srd_t xr = make_srd(x + int64_t(m0) * d.ldx, st < k1 ? uint32_t(mrows * d.ldx * 2) : 0u);
    const uint32_t xdst = stage + Cfg::kABytes;
#pragma unroll
    for (int i = 0; i < Cfg::kXLoads; ++i) {
      const int j = wave * Cfg::kXLoads + i;
      const int row = 8 * j + (lane >> 3);
      const int c8 = (lane & 7) ^ ((row >> 1) & 7);
      dma16<false>(xr, xdst + j * 1024, int(row * d.ldx * 2) + st * 128 + c8 * 16);
    }
    // metadata words of the four slabs (sparse tiles only)
    const char* mbase = reinterpret_cast<const char*>(meta) + (int64_t(slot) * (tile / 16) + int64_t(rs0) * B2) * 2;
    const srd_t mr = make_srd((live && !is_dense) ? mbase : nullptr, (live && !is_dense) ? 8 * B2 : 0);
    const uint32_t mdst = stage + Cfg::kABytes + Cfg::kXBytes + wn * Cfg::kMetaPerGroup;
#pragma unroll
    for (int i = 0; i < Cfg::kMetaLoads; ++i) {
      // piece wm * kMetaLoads + i of the group's metadata (past the end: an
      // empty out-of-range load that keeps the per-step count constant)
      const int piece = wm * Cfg::kMetaLoads + i;
      const bool real = piece < Cfg::kMetaPerGroup / 1024;
      dma16<false>(mr, real ? mdst + piece * 1024 : smem_base + STAGES * Cfg::kStage,
                   real ? piece * 1024 + lane * 16 : 0x40000000);
    }
    tis[sg] = ti;
  };

  f32x4_t acc[4][MBW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Every step runs on v_smfmac with the accumulators updated in place.  A
  // sparse slab is one A operand (its stored chunk) with its index word.  A
  // dense 64-column slab is split into two 2:4 operands: positions 0,1 of
  // every group of four (index word 0x4444) and positions 2,3 (0xEEEE).
  // Lane L (row L%16, lane group g) needs the 16 columns 16g..16g+15, held
  // by lane groups 2(g%2) and 2(g%2)+1 of dense chunk g/2; of the two 16-byte
  // reads, dwords 0 and 2 form the first operand and dwords 1 and 3 the
  // second.  Dense steps thus issue two sparse products per slab, the same
  // matrix-core time as two 16x16x32 MFMAs.
  //
  // Both kinds share the first pass (one product per slab and token block)
  // and its accumulator registers; dense steps add the second pass.  Every
  // LDS read is a whole 16-byte read (the 64 lanes of a read cover 1 KiB
  // without bank conflicts); the weight reads are volatile so the compiler
  // cannot split one into dword reads of the shuffled halves (lanes 16 bytes
  // apart reading single dwords conflict four ways).  A sparse step reads its chunk twice (the second read feeds
  // nothing) so that both kinds run the same instructions up to the second
  // pass.
  auto compute = [&](int sg, int32_t st) {
    const int32_t ti = tis[sg];
    if (ti == kNone) return;
    const char* stage = smem_dyn + sg * Cfg::kStage;
    const char* xsrc = stage + Cfg::kABytes;
    const bool is_dense = ti >= 0;
    const char* wbase = stage + wn * 8192;
    const int r_off = is_dense ? (q >> 1) * 1024 + ((2 * (q & 1)) * 16 + (lane & 15)) * 16 : lane * 16;
    const int r_off2 = is_dense ? r_off + 256 : r_off;
    const char* msrc = stage + Cfg::kABytes + Cfg::kXBytes + wn * Cfg::kMetaPerGroup +
                       lane * (B2 / 32) + (st % kStepsPerTile) * 2;
    // all-ones for a dense step; opaque to the optimiser so the selects
    // below stay bit-selects instead of becoming branches (each branch would
    // wait for its slab's reads on its own)
    uint32_t dm = is_dense ? ~0u : 0u;
    asm("" : "+v"(dm));
    uint4 a0[4], a1[4];
    uint32_t i0[4];
    if constexpr (META == HYB_META_MASK8) {
      // 4:8: the sparse chunk's two groups per lane, expanded, stand in for
      // the dense slab's two pieces; every step runs both passes.
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const u32x4_t v0 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off);
        const u32x4_t v1 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off2);
        const uint32_t m = *reinterpret_cast<const uint16_t*>(msrc + sl * 2 * B2);
        uint32_t e[8];
        expand8_lane(lut8, v0[0], v0[1], v0[2], v0[3], m, e);
        const uint32_t l0 = bitsel(dm, v0[0], e[0]), l1 = bitsel(dm, v0[1], e[1]);
        const uint32_t l2 = bitsel(dm, v0[2], e[2]), l3 = bitsel(dm, v0[3], e[3]);
        const uint32_t h0 = bitsel(dm, v1[0], e[4]), h1 = bitsel(dm, v1[1], e[5]);
        const uint32_t h2 = bitsel(dm, v1[2], e[6]), h3 = bitsel(dm, v1[3], e[7]);
        a0[sl] = make_uint4(l0, l2, h0, h2);
        a1[sl] = make_uint4(l1, l3, h1, h3);
      }
      uint4 bq[MBW][2];
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) {
        const int row = (wm * MBW + mb) * 16 + (lane & 15);
        const int sw = (row >> 1) & 7;
        bq[mb][0] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + ((q ^ sw) * 16));
        bq[mb][1] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + (((q + 4) ^ sw) * 16));
      }
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[sl][mb] = smfmac16x16x64<DT>(a0[sl], bq[mb][0], bq[mb][1], 0x4444u, acc[sl][mb]);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[sl][mb] = smfmac16x16x64<DT>(a1[sl], bq[mb][0], bq[mb][1], 0xEEEEu, acc[sl][mb]);
      return;
    }
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const u32x4_t v0 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off);
      const u32x4_t v1 = *(const volatile lds_u32x4_t*)(wbase + (2 * sl) * 1024 + r_off2);
      const uint32_t m = *reinterpret_cast<const uint16_t*>(msrc + sl * 2 * B2);
      a0[sl] = make_uint4(v0[0], bitsel(dm, v0[2], v0[1]), bitsel(dm, v1[0], v0[2]), bitsel(dm, v1[2], v0[3]));
      a1[sl] = make_uint4(v0[1], v0[3], v1[1], v1[3]);
      i0[sl] = bitsel(dm, 0x4444u, idx2_word<META>(m));
    }
    uint4 bq[MBW][2];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      const int row = (wm * MBW + mb) * 16 + (lane & 15);
      const int sw = (row >> 1) & 7;
      bq[mb][0] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + ((q ^ sw) * 16));
      bq[mb][1] = *reinterpret_cast<const uint4*>(xsrc + row * 128 + (((q + 4) ^ sw) * 16));
    }
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        acc[sl][mb] = smfmac16x16x64<DT>(a0[sl], bq[mb][0], bq[mb][1], i0[sl], acc[sl][mb]);
    if (is_dense) {
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
          acc[sl][mb] = smfmac16x16x64<DT>(a1[sl], bq[mb][0], bq[mb][1], 0xEEEEu, acc[sl][mb]);
    }
  };

  // Prologue: steps 0 .. STAGES-2.
#pragma unroll
  for (int sg = 0; sg < STAGES - 1; ++sg) issue(k0 + sg, sg, tile_index(k0 + sg));
  for (int32_t s0 = k0; s0 < k1; s0 += STAGES) {
#pragma unroll
    for (int sg = 0; sg < STAGES; ++sg) {
      const int32_t st = s0 + sg;
      // Step st's loads are complete once at most the STAGES-2 later steps'
      // loads are outstanding; the barrier makes every wavefront's DMA
      // writes visible and frees the stage read in the previous step.
      wait_vmcnt<(STAGES - 2) * Cfg::kLoadsPerStep>();
      __syncthreads();
      constexpr int kAhead = STAGES - 1;
      issue(st + kAhead, (sg + kAhead) % STAGES, tile_index(st + kAhead));
      if (st < k1) compute(sg, st);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < MBW; ++j) acc_out[i][j] = acc[i][j];
}

// Stores a wavefront's outputs of an LDS-fed tile (lane L: rows
// n0 + 16 sl + 4 (L/16) + 0..3, token mt0 + 16 mb + L%16), adding the
// low-rank term first when `lr` is set.
template <int DT, int MBW>
__device__ __forceinline__ void lds_store(f32x4_t (&acc)[4][MBW], void* y, const GemmDims& d, int32_t n0,
                                          int32_t mt0, bool lr) {
  const int lane = threadIdx.x & 63;
  if (n0 >= d.n) return;
  if (lr && d.rank > 0) lr_block<DT, 4, MBW>(acc, d, n0, mt0, lane);
  const bool vec_ok = y_vec_ok(y, d);
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    const int64_t m = int64_t(mt0) + mb * 16 + (lane & 15);
    if (m >= d.m) continue;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) store_row4(y, d, m, int64_t(n0) + sl * 16 + (lane >> 4) * 4, acc[sl][mb], vec_ok);
  }
}

template <int B2, int DT, int META, int MB, int STAGES, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_lds(const uint4* __restrict__ dense,
                                                  const uint4* __restrict__ val,
                                                  const uint16_t* __restrict__ meta,
                                                  const int32_t* __restrict__ tidx,
                                                  const uint16_t* __restrict__ x,
                                                  void* __restrict__ y, GemmDims d) {
  using Cfg = GemmLdsCfg<B2, MB, STAGES, WAVES>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int32_t nb, mbk;
  xcd_grouped_block((d.n + 255) / 256, nb, mbk);
  f32x4_t acc[4][Cfg::kMBW];
  lds_piece<B2, DT, META, MB, STAGES, WAVES>(dense, val, meta, tidx, x, d, nb, mbk, 0, d.tiles_k * (B2 / 64), acc);
  lds_store<DT, Cfg::kMBW>(acc, y, d, nb * 256 + (wave % 4) * 64, mbk * 16 * MB + (wave / 4) * Cfg::kMBW * 16,
                           true);
}

// The LDS-fed 256-row shape with K split across workgroups, on the schedule
// of k_gemm_split (units u = nb * S + k of each token block, G' ranges per
// token block, workgroup w = j * gm + mb, XCD-major).  A partial piece's
// outputs go to workspace slot 2w (the piece the range starts in) or 2w + 1,
// each wavefront writing its own outputs.
template <int B2, int DT, int META, int MB, int STAGES, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_lds_split(const uint4* __restrict__ dense,
                                                        const uint4* __restrict__ val,
                                                        const uint16_t* __restrict__ meta,
                                                        const int32_t* __restrict__ tidx,
                                                        const uint16_t* __restrict__ x, void* __restrict__ y,
                                                        GemmDims d, SplitPlan p, float* __restrict__ ws) {
  using Cfg = GemmLdsCfg<B2, MB, STAGES, WAVES>;
  constexpr int MBW = Cfg::kMBW;
  constexpr int kWave = 4 * MBW * 64 * 4;     // floats of one wavefront's outputs
  constexpr int kPart = WAVES * kWave;        // floats of one piece (256 rows x 16 MB tokens)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t G = int32_t(gridDim.x), L = int32_t(blockIdx.x);
  const int32_t xcd = L % kSplitXcds, per = G / kSplitXcds, extra = G % kSplitXcds;
  const int32_t w = xcd * per + (xcd < extra ? xcd : extra) + L / kSplitXcds;
  const int32_t j = w / p.gm, mbk = w - j * p.gm;
  const int32_t u1 = split_begin(j + 1, p);
  const int32_t n_wave = (wave % 4) * 64, mt0 = mbk * 16 * MB + (wave / 4) * MBW * 16;
  int slot = 0;
  for (int32_t u = split_begin(j, p); u < u1; ++slot) {
    const int32_t nb = u / p.steps;
    const int32_t ts = nb * p.steps;
    const int32_t k0 = u - ts;
    const int32_t k1 = (u1 < ts + p.steps ? u1 : ts + p.steps) - ts;
    f32x4_t acc[4][MBW];
    lds_piece<B2, DT, META, MB, STAGES, WAVES>(dense, val, meta, tidx, x, d, nb, mbk, k0, k1, acc);
    if (k0 == 0 && k1 == p.steps) {
      lds_store<DT, MBW>(acc, y, d, nb * 256 + n_wave, mt0, true);
    } else {
      if (k0 == 0 && d.rank > 0 && nb * 256 + n_wave < d.n) lr_block<DT, 4, MBW>(acc, d, nb * 256 + n_wave, mt0, lane);
      float* part = ws + (2 * int64_t(w) + (slot == 0 ? 0 : 1)) * kPart + wave * kWave;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
          *reinterpret_cast<f32x4_t*>(part + ((sl * MBW + mb) * 64 + lane) * 4) = acc[sl][mb];
    }
    u = ts + k1;
  }
}

// k_gemm_split_sum for the LDS-fed pieces: float4 f of a piece is wavefront
// f / (4 MBW 64), slab (f / (MBW 64)) % 4, token block (f / 64) % MBW, lane
// f % 64.
template <int MB, int WAVES>
__global__ __launch_bounds__(256) void k_gemm_lds_split_sum(const float* __restrict__ ws, void* __restrict__ y,
                                                            GemmDims d, SplitPlan p) {
  constexpr int MBW = MB / (WAVES / 4);
  constexpr int kVec = WAVES * 4 * MBW * 64;  // float4 per piece
  constexpr int kBlocks = kVec / 256;
  const int32_t t = int32_t(blockIdx.x) / kBlocks;
  const int32_t nb = t / p.gm, mt = t - nb * p.gm;
  const int32_t ts = nb * p.steps;
  const int32_t ja = split_owner(ts, p), jb = split_owner(ts + p.steps - 1, p);
  if (ja == jb) return;
  const int f = (int(blockIdx.x) % kBlocks) * 256 + int(threadIdx.x);
  const int64_t first = 2 * (int64_t(ja) * p.gm + mt) + (split_begin(ja, p) >= ts ? 0 : 1);
  f32x4_t s = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(ws + (first * kVec + f) * 4));
  for (int32_t jj = ja + 1; jj <= jb; ++jj)
    s += __builtin_nontemporal_load(
        reinterpret_cast<const f32x4_t*>(ws + (2 * (int64_t(jj) * p.gm + mt) * kVec + f) * 4));
  const int lane = f & 63;
  const int mb = (f >> 6) % MBW;
  const int sl = ((f >> 6) / MBW) & 3;
  const int wave = (f >> 6) / (4 * MBW);
  const int32_t n0 = nb * 256 + (wave % 4) * 64;
  const int64_t m = int64_t(mt) * 16 * MB + ((wave / 4) * MBW + mb) * 16 + (lane & 15);
  if (m >= d.m || n0 >= d.n) return;
  store_row4(y, d, m, int64_t(n0) + sl * 16 + (lane >> 4) * 4, s, y_vec_ok(y, d));
}


// The 256-row LDS tile with K cut into `parts` equal parts, one workgroup
// per (tile, part): part p of tile (nb, mbk) covers K steps
// [p S / parts, (p + 1) S / parts) and writes its partial outputs to
// workspace slot (nb * parts + p) * gm + mbk, each wavefront its own.
// With one piece per workgroup no state lives across pieces, so the larger
// tiles keep the plain kernel's registers.  Logical ids are XCD-major (as in
// k_gemm_split) and run over (part, row block, token block): the gm token
// blocks of one (row block, part) read the same weights at the same K steps
// on one XCD, and the row blocks an XCD holds mostly share its parts, so X
// columns outside them stay out of its L2 (2-5% faster than row block
// before part, bitwise the same sums).
template <int B2, int DT, int META, int MB, int STAGES, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_lds_parts(const uint4* __restrict__ dense,
                                                        const uint4* __restrict__ val,
                                                        const uint16_t* __restrict__ meta,
                                                        const int32_t* __restrict__ tidx,
                                                        const uint16_t* __restrict__ x, GemmDims d, int32_t gm,
                                                        int32_t steps, int32_t parts, float* __restrict__ ws) {
  using Cfg = GemmLdsCfg<B2, MB, STAGES, WAVES>;
  constexpr int MBW = Cfg::kMBW;
  constexpr int kWave = 4 * MBW * 64 * 4;     // floats of one wavefront's outputs
  constexpr int kPart = WAVES * kWave;        // floats of one piece (256 rows x 16 MB tokens)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t G = int32_t(gridDim.x), L = int32_t(blockIdx.x);
  const int32_t xcd = L % kSplitXcds, per = G / kSplitXcds, extra = G % kSplitXcds;
  const int32_t w = xcd * per + (xcd < extra ? xcd : extra) + L / kSplitXcds;
  const int32_t r = w / gm, mbk = w - r * gm;
  const int32_t gn = int32_t(gridDim.x) / (gm * parts);
  const int32_t part = r / gn, nb = r - part * gn;
  const int32_t slot = (nb * parts + part) * gm + mbk;
  const int32_t k0 = int32_t(int64_t(part) * steps / parts), k1 = int32_t(int64_t(part + 1) * steps / parts);
  f32x4_t acc[4][MBW];
  lds_piece<B2, DT, META, MB, STAGES, WAVES>(dense, val, meta, tidx, x, d, nb, mbk, k0, k1, acc);
  const int32_t n0 = nb * 256 + (wave % 4) * 64;
  if (k0 == 0 && d.rank > 0 && n0 < d.n) lr_block<DT, 4, MBW>(acc, d, n0, mbk * 16 * MB + (wave / 4) * MBW * 16, lane);
  float* out = ws + int64_t(slot) * kPart + wave * kWave;
#pragma unroll
  for (int sl = 0; sl < 4; ++sl)
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
      *reinterpret_cast<f32x4_t*>(out + ((sl * MBW + mb) * 64 + lane) * 4) = acc[sl][mb];
}

// Adds the `parts` partial tiles of k_gemm_lds_parts in part order and
// stores the outputs; float4 f of a piece as in k_gemm_lds_split_sum.
template <int MB, int WAVES>
__global__ __launch_bounds__(256) void k_gemm_lds_parts_sum(const float* __restrict__ ws, void* __restrict__ y,
                                                            GemmDims d, int32_t gm, int32_t parts) {
  constexpr int MBW = MB / (WAVES / 4);
  constexpr int kVec = WAVES * 4 * MBW * 64;  // float4 per piece
  constexpr int kBlocks = kVec / 256;
  const int32_t t = int32_t(blockIdx.x) / kBlocks;
  const int32_t nb = t / gm, mt = t - nb * gm;
  const int f = (int(blockIdx.x) % kBlocks) * 256 + int(threadIdx.x);
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(ws) + (int64_t(nb) * parts * gm + mt) * kVec + f;
  f32x4_t s = __builtin_nontemporal_load(src);
  for (int32_t p = 1; p < parts; ++p) s += __builtin_nontemporal_load(src + int64_t(p) * gm * kVec);
  const int lane = f & 63;
  const int mb = (f >> 6) % MBW;
  const int sl = ((f >> 6) / MBW) & 3;
  const int wave = (f >> 6) / (4 * MBW);
  const int32_t n0 = nb * 256 + (wave % 4) * 64;
  const int64_t m = int64_t(mt) * 16 * MB + ((wave / 4) * MBW + mb) * 16 + (lane & 15);
  if (m >= d.m || n0 >= d.n) return;
  store_row4(y, d, m, int64_t(n0) + sl * 16 + (lane >> 4) * 4, s, y_vec_ok(y, d));
}

}  // namespace




namespace {

template <int B2, int DT, int META, int MB, int STAGES, int WAVES>
hipError_t gemm_lds_go(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, const SplitArgs& sp,
                       hipStream_t s) {
  using Cfg = GemmLdsCfg<B2, MB, STAGES, WAVES>;
  static_assert(Cfg::kBytes <= 160 * 1024, "LDS budget");
  const int64_t gm = (int64_t(m) + 16 * MB - 1) / (16 * MB);
  const int64_t gn = (L.n + 255) / 256;
  if (gn * gm >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
  if constexpr (MB == 4 || MB == 8) {
    if (sp.groups > 0) {
      // K split over sp.groups workgroups in all, sp.groups / gm per token
      // block (workspace checked by the caller, as for gemm_rx_go)
      const int64_t steps = int64_t(d.tiles_k) * (B2 / 64), units = gn * steps;
      const int64_t per_block = sp.groups / gm;
      if (units >= (int64_t(1) << 31) || units < 1 || per_block < 1) return hipErrorInvalidConfiguration;
      SplitPlan p{};
      p.gm = int32_t(gm);
      p.steps = int32_t(steps);
      p.units = int32_t(units);
      p.groups = int32_t(per_block < units ? per_block : units);
      p.q = p.units / p.groups;
      p.r = p.units % p.groups;
      hipLaunchKernelGGL((k_gemm_lds_split<B2, DT, META, MB, STAGES, WAVES>), dim3(unsigned(p.groups * gm)),
                         dim3(64 * WAVES), size_t(Cfg::kBytes), s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d, p,
                         sp.ws);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((k_gemm_lds_split_sum<MB, WAVES>), dim3(unsigned(gn * gm * (4 * MB))), dim3(256), 0, s,
                         static_cast<const float*>(sp.ws), q.y, d, p);
      return hipGetLastError();
    }
  }
  if constexpr (MB == 12 || MB == 16) {
    if (sp.groups > 0) {
      // The first rows0 row blocks whole, in one plain launch over whole
      // rounds of the CUs; the blocks after them with K cut into
      // sp.groups / (tail gm) equal parts per tile (the route gives a
      // multiple of the tail's tile count; workspace checked by the caller).
      // The tail runs on a view of the matrix that starts at row rows0 * 256:
      // the tile-index rows, the output columns and the low-rank rows move
      // there; the weight streams are addressed through the tile index.
      const int64_t rows0 = sp.rows0;
      if (rows0 < 0 || rows0 >= gn) return hipErrorInvalidConfiguration;
      GemvPtrs qt = q;
      GemmDims dt = d;
      if (rows0 > 0) {
        GemmDims dp = d;
        dp.n = int32_t(rows0 * 256);
        hipLaunchKernelGGL((k_gemm_lds<B2, DT, META, MB, STAGES, WAVES>), dim3(unsigned(rows0 * gm)),
                           dim3(64 * WAVES), size_t(Cfg::kBytes), s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, dp);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t row0 = rows0 * 256;
        qt.tidx = q.tidx + (row0 / d.b1) * d.tiles_k;
        qt.y = static_cast<char*>(q.y) + row0 * (d.ydt == HYB_F32 ? 4 : 2);
        dt.n = int32_t(d.n - row0);
        if (d.rank > 0) dt.u = d.u + row0 * d.ldu;
      }
      const int64_t steps = int64_t(d.tiles_k) * (B2 / 64), tiles = (gn - rows0) * gm;
      const int64_t parts = sp.groups / tiles;
      if (parts < 2 || parts * tiles != sp.groups || steps < parts || tiles * parts >= (int64_t(1) << 31))
        return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((k_gemm_lds_parts<B2, DT, META, MB, STAGES, WAVES>), dim3(unsigned(tiles * parts)),
                         dim3(64 * WAVES), size_t(Cfg::kBytes), s, q.dense, q.val, q.meta, qt.tidx, q.x, dt,
                         int32_t(gm), int32_t(steps), int32_t(parts), sp.ws);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((k_gemm_lds_parts_sum<MB, WAVES>), dim3(unsigned(tiles * (4 * MB))), dim3(256), 0, s,
                         static_cast<const float*>(sp.ws), qt.y, dt, int32_t(gm), int32_t(parts));
      return hipGetLastError();
    }
  }
  // 1-D launch of gn * gm workgroups, mapped to (row block, token block)
  // inside the kernel.
  hipLaunchKernelGGL((k_gemm_lds<B2, DT, META, MB, STAGES, WAVES>), dim3(unsigned(gn * gm)), dim3(64 * WAVES),
                     size_t(Cfg::kBytes), s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d);
  return hipGetLastError();
}

template <int B2, int DT, int META, int MB, int WAVES, int STAGES, int RG = 1>
hipError_t gemm_rx_go(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, const SplitArgs& sp,
                      hipStream_t s) {
  const int64_t gm = (int64_t(m) + 16 * MB - 1) / (16 * MB);
  const int64_t gn = (L.n + 64 * RG - 1) / (64 * RG);
  if (sp.groups > 0) {
    // K split over sp.groups workgroups in all, sp.groups / gm per token
    // block (the caller has checked the workspace against
    // split_workspace_bytes, which covers sp.groups workgroups)
    const int64_t steps = int64_t(d.tiles_k) * (B2 / 64), units = gn * steps;
    const int64_t per_block = sp.groups / gm;
    if (units >= (int64_t(1) << 31) || units < 1 || per_block < 1) return hipErrorInvalidConfiguration;
    SplitPlan p{};
    p.gm = int32_t(gm);
    p.steps = int32_t(steps);
    p.units = int32_t(units);
    p.groups = int32_t(per_block < units ? per_block : units);
    p.q = p.units / p.groups;
    p.r = p.units % p.groups;
    hipLaunchKernelGGL((k_gemm_split<B2, DT, META, MB, WAVES, STAGES, RG>), dim3(unsigned(p.groups * gm)),
                       dim3(64 * WAVES), 0, s, q.dense, q.val, q.meta, q.tidx, q.x, q.y, d, p, sp.ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_split_sum<MB, RG>), dim3(unsigned(gn * gm * (RG * MB))), dim3(256), 0, s,
                       static_cast<const float*>(sp.ws), q.y, d, p);
    return hipGetLastError();
  }
  if (gm > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(gn), unsigned(gm), 1u};
  hipLaunchKernelGGL((k_gemm_rx<B2, DT, META, MB, WAVES, STAGES, RG>), grid, dim3(64 * WAVES), 0, s, q.dense,
                     q.val, q.meta, q.tidx, q.x, q.y, d);
  return hipGetLastError();
}

// Three LDS stages where they fit (with the 4 KiB selector table of 4:8
// tiles), else two.
template <int B2, int MB, int WAVES, int META>
constexpr int lds_stages() {
  return GemmLdsCfg<B2, MB, 3, WAVES>::kBytes + (META == HYB_META_MASK8 ? 4096 : 0) <= 160 * 1024 ? 3 : 2;
}


template <int B2, int DT, int META>
hipError_t gemm_shape(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, const GemmRoute& r,
                      const SplitArgs& sp, hipStream_t s) {
  if (r.kernel == kRouteLds || r.rg == 4) {
    switch (r.mb) {
      case 16: return gemm_lds_go<B2, DT, META, 16, lds_stages<B2, 16, 8, META>(), 8>(L, q, m, d, sp, s);
      case 12: return gemm_lds_go<B2, DT, META, 12, lds_stages<B2, 12, 8, META>(), 8>(L, q, m, d, sp, s);
      case 8: return gemm_lds_go<B2, DT, META, 8, lds_stages<B2, 8, 8, META>(), 8>(L, q, m, d, sp, s);
      default: return gemm_lds_go<B2, DT, META, 4, lds_stages<B2, 4, 8, META>(), 8>(L, q, m, d, sp, s);
    }
  }
  if (r.rg == 2) {
    if (r.mb == 2) return gemm_rx_go<B2, DT, META, 2, 4, 2, 2>(L, q, m, d, sp, s);
    if (r.mb == 3) return gemm_rx_go<B2, DT, META, 3, 4, 2, 2>(L, q, m, d, sp, s);
    return gemm_rx_go<B2, DT, META, 4, 4, 2, 2>(L, q, m, d, sp, s);
  }
  if (r.waves == 4) {
    switch (r.mb) {
      case 1: return gemm_rx_go<B2, DT, META, 1, 4, 2>(L, q, m, d, sp, s);
      case 2: return gemm_rx_go<B2, DT, META, 2, 4, 2>(L, q, m, d, sp, s);
      default: return gemm_rx_go<B2, DT, META, 4, 4, 2>(L, q, m, d, sp, s);
    }
  }
  switch (r.mb) {
    case 1: return gemm_rx_go<B2, DT, META, 1, 8, 2>(L, q, m, d, sp, s);
    case 2: return gemm_rx_go<B2, DT, META, 2, 8, 2>(L, q, m, d, sp, s);
    default: return gemm_rx_go<B2, DT, META, 4, 8, 2>(L, q, m, d, sp, s);
  }
}

template <int DT, int META>
hipError_t gemm_b2(const hyb_layout& L, const GemvPtrs& q, int m, const GemmDims& d, const GemmRoute& r,
                   const SplitArgs& sp, hipStream_t s) {
  switch (L.b2) {
    case 64: return gemm_shape<64, DT, META>(L, q, m, d, r, sp, s);
    case 128: return gemm_shape<128, DT, META>(L, q, m, d, r, sp, s);
    default: return gemm_shape<256, DT, META>(L, q, m, d, r, sp, s);
  }
}

}  // namespace

// Device scratch of hyb_gemm_noalloc's split launches (the partial tiles),
// in place of a workspace: one array per GPU, held from the library's load
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device array: only the address that hipGetSymbolAddress returns
// for the current device may reach a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[kSplitMaxBytes];

hipError_t split_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_gemm(const hyb_layout& L, const hyb_packed& P, const void* x, int m, int64_t ldx,
                       void* y, int y_dtype, int64_t ldy, hipStream_t s, void* ws, size_t ws_bytes,
                       const float* t, int64_t ldt, const void* u, int64_t ldu, int rank) {
  GemvPtrs q{static_cast<const uint4*>(P.dense), static_cast<const uint4*>(P.val),
             static_cast<const uint16_t*>(P.meta), P.tidx, static_cast<const uint16_t*>(x), y};
  GemmDims d{};
  d.ldx = ldx;
  d.ldy = ldy;
  d.n = int32_t(L.n);
  d.m = m;
  d.tiles_k = int32_t(L.tiles_k);
  d.n_dense = int32_t(L.n_dense);
  d.n_sparse = int32_t(L.n_sparse);
  d.b1 = L.b1;
  d.ydt = y_dtype;
  d.t = t;
  d.u = static_cast<const uint16_t*>(u);
  d.ldt = ldt;
  d.ldu = ldu;
  d.rank = rank;
  const GemmRoute r = gemm_route(L, m, device_cus());
  // Without a large enough workspace a split route runs its shape unsplit.
  SplitArgs sp{0, nullptr, 0};
  if (r.kernel == kRouteSplit && ws && ws_bytes >= split_workspace_bytes(r))
    sp = SplitArgs{r.groups, static_cast<float*>(ws), r.rows0};
  if (L.dtype == HYB_BF16) {
    if (L.meta == HYB_META_IDX2) return gemm_b2<HYB_BF16, HYB_META_IDX2>(L, q, m, d, r, sp, s);
    if (L.meta == HYB_META_MASK4) return gemm_b2<HYB_BF16, HYB_META_MASK4>(L, q, m, d, r, sp, s);
    return gemm_b2<HYB_BF16, HYB_META_MASK8>(L, q, m, d, r, sp, s);
  }
  if (L.meta == HYB_META_IDX2) return gemm_b2<HYB_F16, HYB_META_IDX2>(L, q, m, d, r, sp, s);
  if (L.meta == HYB_META_MASK4) return gemm_b2<HYB_F16, HYB_META_MASK4>(L, q, m, d, r, sp, s);
  return gemm_b2<HYB_F16, HYB_META_MASK8>(L, q, m, d, r, sp, s);
}

}  // namespace hyb
