// Multi-query attention straight from the packed angle codes: NQ query tokens per
// sequence (a chunk of prefill, or the draft tokens of a speculative step under
// verification), each attending causally to the cache.
//
// Method: the codec of "TurboAngle: Near-Lossless KV Cache Compression via Uniform
// Angle Quantization" (arXiv 2603.27467), Abstract, consumed without writing a
// dequantised cache, as in single-query decode attention: scores and the value sum stay
// in the rotated domain, and each output row gets one inverse transform.
//
// With M = NQ * G query rows per kv head (G query heads per kv head) the per-tile work
// is a dense [M x d] x [d x 64] product for the scores and [M x 64] x [64 x d] for the
// values, so it runs on the matrix cores (v_mfma_f32_16x16x16f16: fp16 operands, fp32
// accumulation) instead of one FMA per (row, token, pair). A wave streams whole 64-token
// tiles: it rebuilds the tile's rotated keys r^ (cos, sin) as fp16 in LDS (one lane per
// token), multiplies, runs the online softmax on the score fragments, stores the
// probabilities as fp16, rebuilds the rotated values in the same LDS space (one lane
// per pair) and accumulates P V^. Rows of query token j see tokens [0, L - NQ + j + 1).
// Waves merge through LDS; splits of the sequence merge through the workspace, the last
// workgroup of each (batch, kv head) combining them (log-sum-exp) and storing.
#include "kvq_attn_common.h"

namespace kvq {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Waves per workgroup: 8 for 16 rows and 6 for 32 rows (LDS holds six waves' tiles at
// 32 rows); both keep two waves per SIMD, so one wave's LDS round trips overlap another's
// work. The 32-row kernel holds one tile's code planes in registers at a time (key planes
// loaded at the tile's start, value planes once the keys are rebuilt), reads the query
// operands from LDS and scores one 16-row block at a time. At d = 128 it still spills
// some 60-70 registers to scratch, and measured faster so (151 us per Mistral-7B-shaped
// layer at 32 rows) than as four waves with no spill (167 us).
constexpr int mq_waves(int rb) { return rb == 1 ? 8 : 6; }

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __floats2half2_rn(lo, hi));
}
// Four fp16 values from two dwords (low halves first).
__device__ __forceinline__ h4 h4_from(const uint32_t* p) {
  const uint2 u = make_uint2(p[0], p[1]);
  return __builtin_bit_cast(h4, u);
}

// Maximum and sum over the 16 lanes of each DPP row (lanes 16k .. 16k + 15); the
// maximum on float-ordered integers, as wave_max, so the DPP moves fuse into v_max_i32.
__device__ __forceinline__ float row16_max(float x) {
  int i = float_order(__float_as_int(x));
  i = max(i, dpp_i<kDppXor1>(i));
  i = max(i, dpp_i<kDppXor2>(i));
  i = max(i, dpp_i<kDppHalfMirror>(i));
  i = max(i, dpp_i<kDppMirror>(i));
  return __int_as_float(float_order(i));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x + dpp<kDppMirror>(x);
}

// MFMA operand layouts (16x16x16, wave64): lane l holds A[row l % 16][k 4(l/16) .. +3],
// B[k 4(l/16) .. +3][column l % 16] and D[rows 4(l/16) .. +3][column l % 16].
template <int D, int BK, int BV, int RB>
__global__ __launch_bounds__(mq_waves(RB) * 64) void attn_multi_kernel(AttnArgs a,
                                                                   const uint8_t* __restrict__ cache) {
  using GE = Geo<D, BK, BV>;
  constexpr int kMqWaves = mq_waves(RB);
  constexpr int P = D / 2, M = 16 * RB, NS = D / 16;
  constexpr int KROW = P + 1;  // dwords per token row of the key tile (odd: fewer conflicts)
  constexpr int VROW = 33;     // dwords per feature row of the value tile (64 tokens + pad)
  constexpr int PROW = 33;     // dwords per row of the probability tile
  constexpr int TILEW = 64 * KROW > D * VROW ? 64 * KROW : D * VROW;
  constexpr int MERGEW = M * D + 2 * M;  // a wave's (acc, max, sum) for the merge
  constexpr int WAVEW = TILEW > MERGEW ? TILEW : MERGEW;
  constexpr int NKT = 1 << BK, NVT = 1 << BV;
  static_assert(M * D <= WAVEW, "rotated queries are staged in the first wave's space");
  // 16 rows: the query operands live in registers; 32 rows: in LDS as fp16 rows
  constexpr bool QREG = RB == 1;
  constexpr int QROW = D / 2 + 1;  // dwords per fp16 query row (odd: fewer conflicts)
  __shared__ float2 lut_k[NKT], lut_v[NVT];
  __shared__ uint32_t s_qh[QREG ? 1 : M * QROW];
  __shared__ __align__(16) uint32_t s_wave[kMqWaves][WAVEW];
  __shared__ uint32_t s_p[kMqWaves][M * PROW];
  __shared__ int s_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x, bk = blockIdx.y;  // bk = b * hkv + kv head
  const int b = bk / a.hkv, kvh = bk % a.hkv;
  // real rows: row = (query - q0) * G + head, for the launch's queries q0 .. q0 + nqc - 1
  const int G = a.group, NQ = a.nq, Q0 = a.q0, MR = a.nqc * G;
  // this sequence's length (per-sequence lengths are clamped to the planned maximum),
  // its tiles and the splits that cover them; a.nsplit stays the stride of the partials
  const int seq_len = a.seq_lens ? (int)min(a.seq_lens[b], (unsigned)a.seq_len) : a.seq_len;
  const int ntiles = (seq_len + kTile - 1) / kTile;
  const int nsplit = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (split >= nsplit) {
    if (split == 0) {  // an empty sequence: every query row attends to nothing
      for (int idx = tid; idx < MR * D; idx += kMqWaves * 64) {
        const int row = idx / D, e = idx % D;
        const size_t o =
            (((size_t)b * NQ + Q0 + row / G) * a.hq + (size_t)kvh * G + row % G) * D + e;
        if (a.out_f32)
          static_cast<float*>(a.out)[o] = 0.f;
        else
          static_cast<__half*>(a.out)[o] = __float2half(0.f);
      }
    }
    return;
  }
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, ntiles);

  const int vi = min(lane, P - 1);  // value pair of this lane (lanes past P repeat the last)

  // 16 rows: the planes of this wave's next tile are loaded while the current one is
  // processed, and the first tile's are requested before the set-up below, whose work
  // then covers their latency. 32 rows (no room for two tiles' planes in registers):
  // a tile's key planes are loaded at its start and its value planes once the keys are
  // rebuilt, their latency covered by the scores and the other wave of the SIMD. A tile
  // the page table maps to no page reads page 0 and counts as holding no token.
  struct Planes {
    uint32_t ka[GE::WKA], kr[GE::WKR], va[2 * BV], vr[8], ks, vp;
    bool present;
  };
  auto tile_words = [&](int tile, bool* present) {
    const long long off = tile_offset(a.pg, b, kvh, a.hkv, a.tiles_per_seq, tile, GE::BYTES);
    *present = off >= 0;
    return reinterpret_cast<const uint32_t*>(cache + (off >= 0 ? off : 0));
  };
  auto load_key_planes = [&](Planes& t, int tile) {
    const uint32_t* w32 = tile_words(tile, &t.present);
#pragma unroll
    for (int w = 0; w < GE::WKA; ++w) t.ka[w] = w32[w * kTile + lane];
#pragma unroll
    for (int w = 0; w < GE::WKR; ++w) t.kr[w] = w32[GE::OFF_KR / 4 + w * kTile + lane];
    t.ks = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(w32) + GE::OFF_KS)[lane];
  };
  auto load_value_planes = [&](Planes& t, int tile) {
    bool present;
    const uint32_t* w32 = tile_words(tile, &present);
    t.vp = w32[GE::OFF_VP / 4 + lane];
#pragma unroll
    for (int w = 0; w < 2 * BV; ++w) t.va[w] = w32[GE::OFF_VA / 4 + w * P + vi];
#pragma unroll
    for (int w = 0; w < 8; ++w) t.vr[w] = w32[GE::OFF_VR / 4 + w * P + vi];
  };
  constexpr bool DB = RB == 1;  // next tile's planes loaded during the current one
  Planes nxt;
  if (DB && tile_begin + wave < tile_end) {
    load_key_planes(nxt, tile_begin + wave);
    load_value_planes(nxt, tile_begin + wave);
  }

  for (int c = tid; c < NKT; c += kMqWaves * 64) {
    float sn = 0.f, co = 0.f;
    if (c < a.n_k) sincospif(2.0f * (float)c / (float)a.n_k, &sn, &co);
    lut_k[c] = make_float2(co, sn);
  }
  for (int c = tid; c < NVT; c += kMqWaves * 64) {
    float sn = 0.f, co = 0.f;
    if (c < a.n_v) sincospif(2.0f * (float)c / (float)a.n_v, &sn, &co);
    lut_v[c] = make_float2(co, sn);
  }
  // rotated queries (times softmax scale * log2 e) as fp32 [M][D]; padding rows zero
  float* s_q = reinterpret_cast<float*>(s_wave[0]);
  for (int row = wave; row < M; row += kMqWaves) {
    float2 v = make_float2(0.f, 0.f);
    if (row < MR) {
      const size_t qoff = (((size_t)b * NQ + Q0 + row / G) * a.hq + (size_t)kvh * G + row % G) * D;
      v = rotate_query<D>(a, qoff, min(lane, P - 1));
    }
    if (lane < P) reinterpret_cast<float2*>(s_q)[row * P + lane] = v;
  }
  __syncthreads();
  h4 qa[QREG ? RB : 1][QREG ? NS : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float4 f = *reinterpret_cast<const float4*>(s_q + (16 * rb + l16) * D + 16 * s + 4 * g4);
        qa[rb][s] = h4{(_Float16)f.x, (_Float16)f.y, (_Float16)f.z, (_Float16)f.w};
      }
  } else {
    for (int idx = tid; idx < M * P; idx += kMqWaves * 64) {
      const float2 f = reinterpret_cast<const float2*>(s_q)[idx];
      s_qh[(idx / P) * QROW + idx % P] = pack_h2(f.x, f.y);
    }
  }
  // tokens visible to each accumulator row of this lane (0 for padding rows)
  int lim[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * rb + 4 * g4 + r;
      lim[rb][r] = row < MR ? seq_len - NQ + Q0 + row / G + 1 : 0;
    }
  __syncthreads();  // the query staging space becomes the first wave's tile space

  f4 o[RB][NS];
  float m_run[RB][4], l_run[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int s = 0; s < NS; ++s) o[rb][s] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_run[rb][r] = -INFINITY;
      l_run[rb][r] = 0.f;
    }
  }
  uint32_t* kb = s_wave[wave];
  uint32_t* pb = s_p[wave];

  for (int tile = tile_begin + wave; tile < tile_end; tile += kMqWaves) {
    Planes cur;
    if constexpr (DB) {
      cur = nxt;
      if (tile + kMqWaves < tile_end) {
        load_key_planes(nxt, tile + kMqWaves);
        load_value_planes(nxt, tile + kMqWaves);
      }
    } else {
      load_key_planes(cur, tile);
    }
    const bool present = cur.present;
    const uint32_t(&ka)[GE::WKA] = cur.ka;
    const uint32_t(&kr)[GE::WKR] = cur.kr;
    const uint32_t(&va)[2 * BV] = cur.va;
    const uint32_t(&vr)[8] = cur.vr;
    const uint16_t ks = (uint16_t)cur.ks;
    const bool tvalid = cur.present && tile * kTile + lane < seq_len;

    // ---- key tile K^[token][feature] (fp16, rotated domain, radius s / 255 * code)
    {
      const float ksc = tvalid ? __half2float(__ushort_as_half(ks)) * (1.0f / 255.0f) : 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const float2 cs = lut_k[field<BK>(ka, i)];
        const float r = (float)((kr[i >> 2] >> (8 * (i & 3))) & 0xFFu) * ksc;
        kb[lane * KROW + i] = pack_h2(r * cs.x, r * cs.y);
        if (!DB && (i & 15) == 15) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!DB) load_value_planes(cur, tile);
    const uint32_t vp = cur.vp;
    __builtin_amdgcn_wave_barrier();

    // ---- per 16-row block: scores S = q~ K^T (fragment [blk] holds rows
    // 16 rb + 4 g4 + r, token 16 blk + l16), then the online softmax per row (base 2),
    // probabilities to LDS as fp16 [row][token]
    _Float16* ph = reinterpret_cast<_Float16*>(pb);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f4 sc[4];
      if constexpr (QREG) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          h4 kv[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s) kv[s] = h4_from(kb + (16 * blk + l16) * KROW + 8 * s + 2 * g4);
          f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[rb][s], kv[s], acc, 0, 0, 0);
          sc[blk] = acc;
        }
      } else {
        // one query fragment per feature block, read from LDS, serves the four token blocks
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) sc[blk] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const h4 qv = h4_from(s_qh + (16 * rb + l16) * QROW + 8 * s + 2 * g4);
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) {
            const h4 kv = h4_from(kb + (16 * blk + l16) * KROW + 8 * s + 2 * g4);
            sc[blk] = __builtin_amdgcn_mfma_f32_16x16x16f16(qv, kv, sc[blk], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v[4], mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          const int t = tile * kTile + 16 * blk + l16;
          v[blk] = present && t < lim[rb][r] ? sc[blk][r] : -INFINITY;
          mx = fmaxf(mx, v[blk]);
        }
        mx = row16_max(mx);
        const float mnew = fmaxf(m_run[rb][r], mx);
        const bool none = mnew == -INFINITY;  // no visible token yet
        const float alpha = none ? 1.f : fast_exp2(m_run[rb][r] - mnew);
        float ps = 0.f;
        const int row = 16 * rb + 4 * g4 + r;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          const float p = none ? 0.f : fast_exp2(v[blk] - mnew);
          ps += p;
          ph[row * (2 * PROW) + 16 * blk + l16] = (_Float16)p;
        }
        l_run[rb][r] = l_run[rb][r] * alpha + ps;
        m_run[rb][r] = mnew;
#pragma unroll
        for (int s = 0; s < NS; ++s) o[rb][s][r] *= alpha;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- value tile V^[feature][token] in the key tile's space (its reads are done):
    // lane = pair; the token's radius parameters come from lane t by readlane
    {
      float r0 = 0.f, beta = 0.f;
      {
        const float smin = __half2float(__ushort_as_half((uint16_t)(vp & 0xFFFFu)));
        const float smax = __half2float(__ushort_as_half((uint16_t)(vp >> 16)));
        r0 = smax;
        if (smax > smin) {
          r0 = smin;
          beta = (__log2f(smax) - __log2f(smin)) * (1.0f / 15.0f);
        }
        if (!tvalid) {
          r0 = 0.f;
          beta = 0.f;
        }
      }
      const bool store = lane < P;
      float x0 = 0.f, y0 = 0.f;
#pragma unroll
      for (int t = 0; t < kTile; ++t) {
        const float r0t = readlane_f(r0, t), bt = readlane_f(beta, t);
        const uint32_t nib = (vr[t >> 3] >> (4 * (t & 7))) & 0xFu;
        const float rr = r0t * fast_exp2((float)nib * bt);
        const float2 cs = lut_v[field<BV>(va, t)];
        const float x = rr * cs.x, y = rr * cs.y;
        if (t & 1) {
          if (store) {
            kb[(2 * vi) * VROW + (t >> 1)] = pack_h2(x0, x);
            kb[(2 * vi + 1) * VROW + (t >> 1)] = pack_h2(y0, y);
          }
        } else {
          x0 = x;
          y0 = y;
        }
        // 32 rows: the scheduler may not gather all of the loop's table reads up front
        if (!DB && (t & 15) == 15) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- O += P V^
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      h4 pa[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) pa[rb] = h4_from(pb + (16 * rb + l16) * PROW + 8 * k4 + 2 * g4);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const h4 vb = h4_from(kb + (16 * s + l16) * VROW + 8 * k4 + 2 * g4);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][s] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa[rb], vb, o[rb][s], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the waves: each writes (acc [M][D], max [M], sum [M]) to its space
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) l_run[rb][r] = row16_sum(l_run[rb][r]);
  __syncthreads();
  float* mine = reinterpret_cast<float*>(s_wave[wave]);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) mine[(16 * rb + 4 * g4 + r) * D + 16 * s + l16] = o[rb][s][r];
  if (l16 == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mine[M * D + 16 * rb + 4 * g4 + r] = m_run[rb][r];
        mine[M * D + M + 16 * rb + 4 * g4 + r] = l_run[rb][r];
      }
  }
  __syncthreads();
  const bool single = nsplit == 1;
  float* s_out = reinterpret_cast<float*>(s_p);  // normalised rows when single: [M][D]
  static_assert(M * D <= kMqWaves * M * PROW, "output staging fits the probability space");
  for (int idx = tid; idx < MR * D; idx += kMqWaves * 64) {
    const int row = idx / D, e = idx % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kMqWaves; ++w)
      mm = fmaxf(mm, reinterpret_cast<const float*>(s_wave[w])[M * D + row]);
    float ll = 0.f, aa = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kMqWaves; ++w) {
        const float* f = reinterpret_cast<const float*>(s_wave[w]);
        const float c = fast_exp2(f[M * D + row] - mm);  // 0 for a wave that saw nothing
        ll += f[M * D + M + row] * c;
        aa += f[row * D + e] * c;
      }
    }
    if (single) {
      s_out[idx] = ll > 0.f ? aa / ll : 0.f;
    } else {
      const size_t rowi = ((size_t)bk * a.nsplit + split) * M + row;
      __hip_atomic_store(a.part_acc + rowi * D + e, aa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (e == 0) {
        __hip_atomic_store(a.part_ml + 2 * rowi, mm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.part_ml + 2 * rowi + 1, ll, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (!single) {
    // the last workgroup of this (batch, kv head) to finish combines the splits; the
    // partials are written and read as agent-scope atomics (device-coherent cache
    // policy), the stores are performed before the ticket is taken (waitcnt, then the
    // barrier) and the ticket is a system-scope atomic: the same ordering argument as
    // the decode-attention kernel's merge
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned t = __hip_atomic_fetch_add(a.tickets + bk, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_SYSTEM);
      s_flag = t == (unsigned)(nsplit - 1);
    }
    __syncthreads();
    if (!s_flag) return;
    for (int idx = tid; idx < MR * D; idx += kMqWaves * 64) {
      const int row = idx / D, e = idx % D;
      // eight splits' loads in flight per round (the partials come from other XCDs
      // through memory)
      auto ld = [](const float* p) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };
      float mm = -INFINITY, ll = 0.f, aa = 0.f;
      for (int s0 = 0; s0 < nsplit; s0 += 8) {
        float mv[8], lv[8], av[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const size_t rowi = ((size_t)bk * a.nsplit + min(s0 + u, nsplit - 1)) * M + row;
          mv[u] = ld(a.part_ml + 2 * rowi);
          lv[u] = ld(a.part_ml + 2 * rowi + 1);
          av[u] = ld(a.part_acc + rowi * D + e);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (s0 + u < nsplit && mv[u] != -INFINITY) {  // skip splits that saw no token
            const float mnew = fmaxf(mm, mv[u]);
            const float c0 = fast_exp2(mm - mnew), c1 = fast_exp2(mv[u] - mnew);
            ll = ll * c0 + lv[u] * c1;
            aa = aa * c0 + av[u] * c1;
            mm = mnew;
          }
        }
      }
      s_out[idx] = ll > 0.f ? aa / ll : 0.f;
    }
    if (tid == 0)
      __hip_atomic_store(a.tickets + bk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  __syncthreads();
  // inverse transform and sign per output row (one wave per row, lane = pair)
  for (int row = wave; row < MR; row += kMqWaves) {
    if (lane < P) {
      const float2 v = reinterpret_cast<const float2*>(s_out)[row * P + lane];
      const size_t ooff = (((size_t)b * NQ + Q0 + row / G) * a.hq + (size_t)kvh * G + row % G) * D;
      store_output<D>(a, ooff, lane, v.x, v.y);
    }
  }
}

}  // namespace

hipError_t launch_attn_multi(const AttnArgs& a, int d, int rows, const uint8_t* cache,
                             hipStream_t stream) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.batch * a.hkv));
  const int rb = rows <= 16 ? 1 : 2;
  const dim3 block(mq_waves(rb) * 64);
#define KVQ_MQ(D_, BK_, BV_, RB_)                                                             \
  if (d == D_ && a.bk == BK_ && a.bv == BV_ && rb == RB_) {                                   \
    hipLaunchKernelGGL((attn_multi_kernel<D_, BK_, BV_, RB_>), grid, block, 0, stream, a, cache); \
    return hipGetLastError();                                                                 \
  }
#define KVQ_MQ_BV(D_, BK_, RB_) KVQ_MQ(D_, BK_, 6, RB_) KVQ_MQ(D_, BK_, 7, RB_) KVQ_MQ(D_, BK_, 8, RB_)
#define KVQ_MQ_BK(D_, RB_) KVQ_MQ_BV(D_, 6, RB_) KVQ_MQ_BV(D_, 7, RB_) KVQ_MQ_BV(D_, 8, RB_)
  KVQ_MQ_BK(64, 1)
  KVQ_MQ_BK(128, 1)
  KVQ_MQ_BK(64, 2)
  KVQ_MQ_BK(128, 2)
#undef KVQ_MQ_BK
#undef KVQ_MQ_BV
#undef KVQ_MQ
  return hipErrorInvalidValue;
}

}  // namespace kvq
