// Decode attention straight from the packed angle codes.
//
// Method: the codec of "TurboAngle: Near-Lossless KV Cache Compression via Uniform
// Angle Quantization" (arXiv 2603.27467), Abstract, consumed without writing a
// dequantised cache (the fused-reconstruction point made in "OCTOPUS: Joint Triplet
// Quantization for KV Cache via Octahedral Parametrization", Why it matters).
//
// The transform R = H diag(sign) / sqrt(d) is orthogonal, so with q~ = R q and
// y^_j the rotated-domain reconstruction of key j,
//   <q, k^_j> = <q~, y^_j> = (s_j / 255) sum_i rho_ji (q~_2i cos t_ji + q~_2i+1 sin t_ji)
// and the output is o = R^T (sum_j p_j z^_j) with z^_j the rotated-domain values:
// one inverse transform per output head instead of one per cached token.
//
// One launch: grid (splits, batch * kv heads), each wave streaming whole 64-token tiles
// (12 waves per workgroup with the key table at up to four heads and with both products
// on the matrix cores at d = 128, else 8). The variant (KTM, chosen on the host by attn_mode) sets how scores and the
// value sum are formed:
//   set-up   the workgroup rotates its G query heads (q~ = R q times
//            softmax_scale * log2(e) / 255) and builds cos/sin tables and, with a key
//            table, the score table T[i][code][head] = q~_2i cos + q~_2i+1 sin in LDS
//            (half of it for power-of-two n). The variant with neither (built only
//            for comparisons) has a small prepare kernel write q~ to the workspace
//            first, and its scores read it through scalar loads.
//   keys     one lane per token: one FMA per pair and head against T, or the matrix
//            cores (fp32 4x4x1 products of q~ and the rebuilt key element).
//            Online softmax per wave in base 2.
//   values   on the matrix cores (the defaults): one lane per pair, fp16 products of
//            four tokens' softmax weights and rebuilt level * (cos, sin) per
//            instruction, fp32 sums. Vector variant: lanes are 4 rows x 16 columns,
//            one token per row and step, weights broadcast along the row with DPP,
//            radius levels gathered with a lane permute.
//   append   (the fused decode step) the wave that will read the tile of a sequence's
//            new slot first codes the new token into it, with the append kernel's code,
//            while the other waves stream their tiles.
//   merge    waves merge through LDS. With one split the workgroup normalises,
//            inverse-transforms and stores; otherwise each split writes
//            (max, sum, acc[d]) per head and the last workgroup of the (batch, kv head)
//            to finish combines them (log-sum-exp), inverse-transforms and stores.
//
// The tile loop is bound by VALU issue first (code unpacking, table addressing, the
// score FMAs; a wave64 fp32 instruction occupies a SIMD for four cycles on this chip),
// then by LDS instruction throughput and load latency, not by HBM traffic.
#include "kvq_attn_common.h"
#include "kvq_codec_dev.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------------------- prepare

// Rotated queries into the workspace, for the kernels without a key table (their
// scores read q~ through scalar loads, which must not see data written by the same
// launch). One wave per (batch, query head).
template <int D>
__global__ __launch_bounds__(64) void attn_prepare_kernel(AttnArgs a) {
  constexpr int P = D / 2;
  const int lane = threadIdx.x;
  if (lane >= P) return;
  const size_t off = (size_t)blockIdx.x * D;
  reinterpret_cast<float2*>(a.qrot)[off / 2 + lane] = rotate_query<D>(a, off, lane);
}

// ---------------------------------------------------------------------------- split

// Value lanes: a wave is 4 rows x 16 columns. Row r takes the 16 token slots
// [16r, 16r + 16) of a tile one per step; column c takes P / 16 consecutive pairs.
constexpr int kRows = 4, kCols = 16, kStepTokens = kTile / kRows;

template <int D, int G, int BK, int BV>
struct SplitCfg {
  using GE = Geo<D, BK, BV>;
  static constexpr int P = D / 2;
  static constexpr int NKT = 1 << BK;         // key-table rows per pair (codes < 2^bk)
  static constexpr int PPL = P / kCols;        // value pairs per lane
  // value-angle words per pair covering one row's 16 tokens; odd widths may start
  // half-way into a word and are realigned after loading
  static constexpr int VAW = (BV & 1) ? (kStepTokens * BV + 16 + 31) / 32 : kStepTokens * BV / 32;
  static constexpr int TAB_BYTES = P * NKT * G * 4;
};

// Registers of one tile: key planes in token-per-lane order, value planes in the
// row/column order above.
template <int D, int G, int BK, int BV>
struct TileRegs {
  using C = SplitCfg<D, G, BK, BV>;
  uint32_t ka[C::GE::WKA], kr[C::GE::WKR], ks, vp;
  uint32_t va[C::PPL][C::VAW], vr[C::PPL][2];
};

// Key planes of one tile (lane = token slot); R is either register set below.
template <int D, int BK, int BV, class R>
__device__ __forceinline__ void load_tile_keys(R& t, const uint8_t* tp, int lane) {
  using GE = Geo<D, BK, BV>;
  const uint32_t* w32 = reinterpret_cast<const uint32_t*>(tp);
#pragma unroll
  for (int w = 0; w < GE::WKA; ++w) t.ka[w] = w32[w * kTile + lane];
#pragma unroll
  for (int w = 0; w < GE::WKR; ++w) t.kr[w] = w32[GE::OFF_KR / 4 + w * kTile + lane];
  t.ks = reinterpret_cast<const uint16_t*>(tp + GE::OFF_KS)[lane];
}

// Value planes of one tile in the row/column order of the value lanes, plus the
// per-token radius parameters (lane = token slot).
template <int D, int G, int BK, int BV>
__device__ __forceinline__ void load_tile_values(TileRegs<D, G, BK, BV>& t, const uint8_t* tp,
                                                 int lane, int row, int col) {
  using C = SplitCfg<D, G, BK, BV>;
  using GE = typename C::GE;
  constexpr int P = C::P, PPL = C::PPL;
  const uint32_t* w32 = reinterpret_cast<const uint32_t*>(tp);
  t.vp = w32[GE::OFF_VP / 4 + lane];
  const int w0 = (row * kStepTokens * BV) >> 5;
#pragma unroll
  for (int w = 0; w < C::VAW; ++w) {
    const uint32_t* src = w32 + GE::OFF_VA / 4 + (w0 + w) * P + col * PPL;
    if constexpr (PPL == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      t.va[0][w] = v.x; t.va[1 % PPL][w] = v.y; t.va[2 % PPL][w] = v.z; t.va[3 % PPL][w] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      t.va[0][w] = v.x; t.va[1 % PPL][w] = v.y;
    }
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t* src = w32 + GE::OFF_VR / 4 + (2 * row + w) * P + col * PPL;
    if constexpr (PPL == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      t.vr[0][w] = v.x; t.vr[1 % PPL][w] = v.y; t.vr[2 % PPL][w] = v.z; t.vr[3 % PPL][w] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      t.vr[0][w] = v.x; t.vr[1 % PPL][w] = v.y;
    }
  }
}

// G consecutive floats from LDS (16-byte aligned when G >= 4).
template <int G>
__device__ __forceinline__ void load_row(float (&tv)[G], const float* t) {
  if constexpr (G >= 4) {
#pragma unroll
    for (int g = 0; g < G; g += 4) {
      const float4 v = *reinterpret_cast<const float4*>(t + g);
      tv[g] = v.x; tv[g + 1] = v.y; tv[g + 2] = v.z; tv[g + 3] = v.w;
    }
  } else if constexpr (G == 2) {
    const float2 v = *reinterpret_cast<const float2*>(t);
    tv[0] = v.x; tv[1] = v.y;
  } else {
    tv[0] = t[0];
  }
}

// Broadcast lane 16 * row + k to every lane of its row of 16 (DPP row_newbcast). Every
// source lane is valid, so the bound-control bit only spares a move of the old value.
__device__ __forceinline__ float row_bcast(float v, int k) {
  const int x = __float_as_int(v);
  int r;
  switch (k) {
    case 0: r = __builtin_amdgcn_update_dpp(0, x, 0x150, 0xF, 0xF, true); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x151, 0xF, 0xF, true); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0x152, 0xF, 0xF, true); break;
    case 3: r = __builtin_amdgcn_update_dpp(0, x, 0x153, 0xF, 0xF, true); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, x, 0x154, 0xF, 0xF, true); break;
    case 5: r = __builtin_amdgcn_update_dpp(0, x, 0x155, 0xF, 0xF, true); break;
    case 6: r = __builtin_amdgcn_update_dpp(0, x, 0x156, 0xF, 0xF, true); break;
    case 7: r = __builtin_amdgcn_update_dpp(0, x, 0x157, 0xF, 0xF, true); break;
    case 8: r = __builtin_amdgcn_update_dpp(0, x, 0x158, 0xF, 0xF, true); break;
    case 9: r = __builtin_amdgcn_update_dpp(0, x, 0x159, 0xF, 0xF, true); break;
    case 10: r = __builtin_amdgcn_update_dpp(0, x, 0x15A, 0xF, 0xF, true); break;
    case 11: r = __builtin_amdgcn_update_dpp(0, x, 0x15B, 0xF, 0xF, true); break;
    case 12: r = __builtin_amdgcn_update_dpp(0, x, 0x15C, 0xF, 0xF, true); break;
    case 13: r = __builtin_amdgcn_update_dpp(0, x, 0x15D, 0xF, 0xF, true); break;
    case 14: r = __builtin_amdgcn_update_dpp(0, x, 0x15E, 0xF, 0xF, true); break;
    default: r = __builtin_amdgcn_update_dpp(0, x, 0x15F, 0xF, 0xF, true); break;
  }
  return __int_as_float(r);
}
__device__ __forceinline__ float bperm_f(int byte_addr, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(byte_addr, __float_as_int(v)));
}

// ---------------------------------------------------------------- matrix-core mode
//
// KTM 3 (scores) and bit 2 of KTM (values) run a tile's products on the matrix cores:
// sixteen independent 4x4 blocks per instruction. Lane 4b + i supplies row i of block
// b's A operand, lane 4b + j column j of its B operand, and lane 4b + j receives
// D[b][0..3][j] in its four result registers (checked on the GPU against a host
// product). With the query heads of a kv head as the four rows:
//   scores  v_mfma_f32_4x4x1f32 (fp32, k = 1), lane = token: A = q~[head][e] (lane l
//           holds head l & 3), B = the token's reconstructed rotated key element
//           rho * (cos, sin)[code]; one product per element e leaves the four heads'
//           scores in the token's lane. Kept in fp32: with fp16 keys and queries a CPU
//           emulation over real codes puts the attention error at up to 2e-3 on inputs
//           with outlier channels (large logits).
//   values  v_mfma_f32_4x4x4f16 (fp16 operands, fp32 sums, k = 4 tokens), lane = pair
//           (d = 128) or pair and token half (d = 64): A = the softmax weights of four
//           tokens for head l & 3, B = level(rho) * (cos, sin)[code] of those tokens in
//           the lane's pair (formed in fp32, rounded once to fp16); the rotated-domain
//           sums of the four heads accumulate in the pair's lane. Rounding the operands
//           adds about 2^-11 relative per term, well inside the attention bound.
// The VALU keeps only code unpacking, table lookups and the multiplies per element.
// Rows past G are zero.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4x __attribute__((ext_vector_type(4)));
typedef _Float16 h2x __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma4x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

template <int D, int G, int BK, int BV>
struct MxCfg {
  static constexpr int P = D / 2;
  static constexpr int HG = G > 4 ? G / 4 : 1;         // groups of four heads (rows)
  static constexpr int VT = D == 128 ? 64 : 32;        // value tokens per lane
  static constexpr int VAW = VT * BV / 32;             // value angle words per lane
  static constexpr int VRW = VT / 8;                   // value radius words per lane
  // query operands in registers (128 VGPRs at d = 128), unless the extra words of
  // 8-bit key codes would then spill: then they are read from LDS per pair
  static constexpr bool QREG = HG * D <= 128 && BK < 8;
  static constexpr int PS_HALVES = HG * 4 * kTile;     // per wave: fp16 weights [HG][4][64]
  static constexpr int LEV_HALVES = kTile * 16;        // per wave: fp16 levels [64][16]
  static constexpr int WAVE_BYTES = (PS_HALVES + LEV_HALVES) * 2;
};

// Registers of one tile in matrix-core mode: key planes with lane = token, value planes
// with lane = pair (and token half for d = 64), value parameters with lane = token.
template <int D, int G, int BK, int BV>
struct MxRegs {
  using GE = Geo<D, BK, BV>;
  using M = MxCfg<D, G, BK, BV>;
  uint32_t ka[GE::WKA], kr[GE::WKR], ks, vp;
  uint32_t va[M::VAW], vr[M::VRW];
};

template <int D, int G, int BK, int BV>
__device__ __forceinline__ void load_tile_values_mx(MxRegs<D, G, BK, BV>& t, const uint8_t* tp,
                                                    int lane) {
  using GE = Geo<D, BK, BV>;
  using M = MxCfg<D, G, BK, BV>;
  constexpr int P = D / 2;
  const uint32_t* w32 = reinterpret_cast<const uint32_t*>(tp);
  const int pr = lane & (P - 1), th = D == 128 ? 0 : lane >> 5;
  t.vp = w32[GE::OFF_VP / 4 + lane];
#pragma unroll
  for (int w = 0; w < M::VAW; ++w) t.va[w] = w32[GE::OFF_VA / 4 + (th * M::VAW + w) * P + pr];
#pragma unroll
  for (int w = 0; w < M::VRW; ++w) t.vr[w] = w32[GE::OFF_VR / 4 + (th * M::VRW + w) * P + pr];
}

// Waves per split workgroup (attn_waves): 12 (three per SIMD) with the key table at up to
// four heads per kv head, and with both products on the matrix cores at d = 128 (both stay
// under 168 VGPRs); 8 otherwise (KTM 3 keeps the query operands in 128 VGPRs).
constexpr int split_waves(int ktm, int group, int d) { return attn_waves(ktm, group, d); }

// One workgroup per (split, batch * kv head). KTM (key-table mode) 1: scores read a
// per-workgroup table T[i][c][h] = q~_h,2i cos(2 pi c / n) + q~_h,2i+1 sin(2 pi c / n)
// from LDS, one FMA per (pair, head). KTM 2 (n a power of two): only rows c < n/2 are
// stored and T[i][c + n/2] = -T[i][c] (the angle plus pi), the top code bit flipping the
// sign of the radius; half the LDS and fewer bank conflicts for one extra operation per
// pair, and it leaves room for the matrix-core value rows beside 8-bit codes at up to two
// heads. KTM 0: scores use the cos/sin table and the rotated query from scalar registers.
// Lazy softmax maximum: a tile's scores may exceed the running maximum by up to this
// (base-2 units) before it is refreshed, so the weights stay within 2^8.
constexpr float kLazyLog2 = 8.f;

template <int D, int G, int BK, int BV, int KTM>
__global__ __launch_bounds__(split_waves(KTM, G, D) * 64) void attn_decode_kernel(
    AttnArgs a, const uint8_t* __restrict__ cache, const float* __restrict__ qrot,
    AppendArgs app) {
  using C = SplitCfg<D, G, BK, BV>;
  using GE = typename C::GE;
  using M = MxCfg<D, G, BK, BV>;
  // Key mode (KTM & 3): 0 scalar-loaded query, 1 full score table, 2 half score table,
  // 3 matrix cores; bit 2 of KTM: values on the matrix cores. KT: the query is rotated
  // in the kernel; TAB: scores from the LDS score table.
  constexpr int KMODE = KTM & 3;
  constexpr bool KT = KMODE != 0, HALF = KMODE == 2, MXK = KMODE == 3, TAB = KT && !MXK;
  constexpr bool MXV = (KTM & 4) != 0, MX = MXK || MXV;
  // lazy softmax maximum where the wave maxima of eight or more heads per tile are a
  // visible cost (4-5% of the 70B-shaped layers' time); the table kernels keep the
  // branch-free form, whose score pipeline the compiler otherwise breaks up
  constexpr bool LAZY = MXK && G > 4;
  constexpr int P = C::P, NKT = C::NKT, PPL = C::PPL, NW = split_waves(KTM, G, D);
  constexpr int NTAB = HALF ? NKT / 2 : NKT;  // table rows per pair
  // LDS used during the tile loop: the score table, then the waves' value rows
  constexpr int TABLE_BYTES = TAB ? P * NTAB * G * 4 : 0;
  constexpr int TAB_BYTES = TABLE_BYTES + (MXV ? NW * M::WAVE_BYTES : 0);
  constexpr int MERGE_BYTES = NW * G * (D + 2) * 4;
  // With a score table and matrix-core values the tile loop never reads the rotated
  // query, so it lives in the union as well: in the space of the value rows while the
  // table is built (the rows are first written after the barrier that ends the build),
  // and after the merge buffers once the loop is done (normalised output). That leaves
  // room for the full table beside the value rows at four heads and 7-bit codes.
  constexpr bool QU = TAB && MXV;
  constexpr int QB = G * D * 4;
  static_assert(!QU || NW * M::WAVE_BYTES >= QB, "query does not fit in the value rows");
  constexpr int UNION_BYTES =
      TAB_BYTES > MERGE_BYTES + (QU ? QB : 0) ? TAB_BYTES : MERGE_BYTES + (QU ? QB : 0);
  // small cos/sin tables at the bottom of LDS so their lookups fold the base into the
  // instruction's immediate offset; then the rotated query (later the normalised
  // output) unless it lives in the union, a flag, and the key table (or the merge
  // buffers)
  constexpr int LUTK_OFF = 0, LUTV_OFF = NKT * 8, Q_OFF = LUTV_OFF + (1 << BV) * 8;
  constexpr int FLAG_OFF = Q_OFF + (QU ? 0 : QB), UNION_OFF = FLAG_OFF + 16;
  __shared__ __align__(16) char smem[UNION_OFF + UNION_BYTES];
  static_assert(UNION_OFF + UNION_BYTES == attn_lds_bytes(D, G, BK, BV, KTM),
                "LDS layout and its host-side model disagree");
  float2* lut_k = reinterpret_cast<float2*>(smem + LUTK_OFF);
  float2* lut_v = reinterpret_cast<float2*>(smem + LUTV_OFF);
  int* s_flag = reinterpret_cast<int*>(smem + FLAG_OFF);
  char* s_union = smem + UNION_OFF;
  // rotated query [G][D] (set-up, and the matrix-core scores), normalised output [G][D]
  float* s_q = reinterpret_cast<float*>(QU ? s_union + TABLE_BYTES : smem + Q_OFF);
  float* s_out = reinterpret_cast<float*>(QU ? s_union + MERGE_BYTES : smem + Q_OFF);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar tile addresses
  const int row = lane >> 4, col = lane & 15;
  const int split = blockIdx.x, bk = blockIdx.y;  // bk = b * hkv + kv head
  // This entry's length (per-entry lengths are clamped to the planned maximum; with a
  // fused append, the appended slot + 1), its tiles and the splits that cover them;
  // a.nsplit stays the stride of the partials.
  const bool append = app.positions != nullptr;
  const unsigned apos = append ? app.positions[bk / a.hkv] : 0u;
  const int seq_len = append ? (apos >= (unsigned)a.seq_len ? a.seq_len : (int)apos + 1)
                      : a.seq_lens ? (int)min(a.seq_lens[bk / a.hkv], (unsigned)a.seq_len)
                                   : a.seq_len;
  const int ntiles = (seq_len + kTile - 1) / kTile;
  const int nsplit = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (split >= nsplit) {
    if (split == 0) {  // an empty sequence attends to nothing: zero output
      for (int idx = tid; idx < G * D; idx += NW * 64) {
        const size_t o = (size_t)bk * G * D + idx;
        if (a.out_f32)
          static_cast<float*>(a.out)[o] = 0.f;
        else
          static_cast<__half*>(a.out)[o] = __float2half(0.f);
      }
    }
    return;
  }
  // rotated query in the workspace, written by the prepare kernel (only launched when
  // there is no key table: then the scores read it through scalar loads)
  const float* qg = qrot + (size_t)bk * G * D;

  // Set-up order: the query loads go out first (wave g < G loads head kv_head * G + g;
  // query heads of one kv head are consecutive, so its row is bk * G + g), then the
  // first tile's key loads. Loads complete in order, so the query is waited for without
  // waiting for the tile, whose latency overlaps the table build.
  // Both loads are unconditional (indices clamped into range), so no branch separates
  // them from the rotation below and only the query loads are waited for there.
  uint2 qraw = make_uint2(0u, 0u);
  if (KT) qraw = load_query_pair(a, ((size_t)bk * G + min(wave, G - 1)) * D, min(lane, P - 1));
  __builtin_amdgcn_sched_barrier(0);  // keep the query loads ahead of the tile loads
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, ntiles);
  // Tile addresses (wave-uniform): tile t sits at base + t * stride in a contiguous
  // cache, at base + page * stride with page = table[t] in a paged pool. A tile the
  // table maps to no page reads page 0 and counts as holding no token.
  const int* ptab = nullptr;
  const uint8_t* base = cache + (size_t)bk * a.tiles_per_seq * GE::BYTES;
  size_t stride = GE::BYTES;
  if (a.pg.table) {
    const int b = bk / a.hkv;
    ptab = a.pg.table + (size_t)b * a.pg.pages_per_seq;
    base = cache + (size_t)(bk - b * a.hkv) * GE::BYTES;
    stride = (size_t)a.hkv * GE::BYTES;
  }
  // Fused append: the appended token is coded by the wave that reads its tile (for a
  // slot past the attended range, wave 0 of split 0), after the set-up and before that
  // wave's first tile load. Only this workgroup reads the tile in this launch.
  bool owner = false;
  int app_tile = 0;
  if (append && apos < (unsigned)app.capacity) {
    app_tile = (int)(apos / kTile);
    if (app_tile < ntiles) {
      const int s = app_tile / a.tiles_per_split;
      owner = split == s && wave == (app_tile - s * a.tiles_per_split) % NW;
    } else {
      owner = split == 0 && wave == 0;
    }
  }
  std::conditional_t<MXV, MxRegs<D, G, BK, BV>, TileRegs<D, G, BK, BV>> cur;
  int tile = tile_begin + wave;
  auto first_tile_keys = [&]() {
    const int t0 = min(tile, tile_end - 1);
    int idx = t0;
    if (ptab) {
      const int page = ptab[t0];
      idx = page >= 0 && page < a.pg.num_pages ? page : 0;
    }
    load_tile_keys<D, BK, BV>(cur, base + idx * stride, lane);
  };
  if (!owner) first_tile_keys();
  if (KT) {
    const float2 qv = rotate_query_pair<D>(a, qraw, lane);
    if (wave < G && lane < P) reinterpret_cast<float2*>(s_q)[wave * P + lane] = qv;
  }

  // cos/sin of the bin centres 2 pi c / n; rows past n are only ever read for slots
  // past the sequence end and are zeroed
  for (int c = tid; c < NKT; c += NW * 64) {
    float sn = 0.f, co = 0.f;
    if (c < a.n_k) sincospif(2.0f * (float)c / (float)a.n_k, &sn, &co);
    lut_k[c] = make_float2(co, sn);
  }
  for (int c = tid; c < (1 << BV); c += NW * 64) {
    float sn = 0.f, co = 0.f;
    if (c < a.n_v) sincospif(2.0f * (float)c / (float)a.n_v, &sn, &co);
    if constexpr (MXV)  // matrix-core values: fp16 pairs, the operand type
      reinterpret_cast<h2x*>(lut_v)[c] = h2x{(_Float16)co, (_Float16)sn};
    else
      lut_v[c] = make_float2(co, sn);
  }
  __syncthreads();
  float* ktab = reinterpret_cast<float*>(s_union);
  if (TAB) {
    // NW*64 threads: each owns one pair (q~ loaded once) and a stride of codes
    constexpr int TPP = NW * 64 / P;  // threads per pair
    const int i = tid / TPP, c0 = tid % TPP;
    float qa[G], qb[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      qa[g] = s_q[g * D + 2 * i];
      qb[g] = s_q[g * D + 2 * i + 1];
    }
    for (int c = c0; c < NTAB; c += TPP) {
      const float2 cs = lut_k[c];
      float tv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) tv[g] = fmaf(qa[g], cs.x, qb[g] * cs.y);
      float* dst = ktab + (i * NTAB + c) * G;
#pragma unroll
      for (int g = 0; g < G; g += (G >= 4 ? 4 : G)) {
        if (G >= 4)
          *reinterpret_cast<float4*>(dst + g) = make_float4(tv[g], tv[(g + 1) % G], tv[(g + 2) % G], tv[(g + 3) % G]);
        else if (G == 2)
          *reinterpret_cast<float2*>(dst) = make_float2(tv[0], tv[1 % G]);
        else
          dst[0] = tv[0];
      }
    }
    __syncthreads();
  }

  if (owner) {
    int idx = app_tile;
    bool present = true;
    if (ptab) {
      const int page = ptab[app_tile];
      present = page >= 0 && page < a.pg.num_pages;
      idx = page;
    }
    if (present) {  // a tile mapped to no page takes no write
      const int b = bk / a.hkv, h = bk - b * a.hkv;
      const size_t esz = app.f32 ? 4 : 2;
      const size_t roff = ((size_t)b * app.sb + (size_t)h * app.sh) * esz;
      CodecArgs c;
      c.n_k = a.n_k;
      c.n_v = a.n_v;
      c.bk = BK;
      c.bv = BV;
      c.inv_sqrt_d = app.inv_sqrt_d;
      c.k_bins_per_rad = app.k_bins_per_rad;
      c.v_bins_per_rad = app.v_bins_per_rad;
      c.sign = a.sign;
      TileGeom g;
      g.ka = 0;
      g.kr = GE::OFF_KR;
      g.ks = GE::OFF_KS;
      g.va = GE::OFF_VA;
      g.vr = GE::OFF_VR;
      g.vp = GE::OFF_VP;
      g.wka = GE::WKA;
      g.wkr = GE::WKR;
      append_token<D>(c, g, const_cast<uint8_t*>(base) + idx * stride, (int)(apos % kTile),
                      static_cast<const char*>(app.k) + roff,
                      static_cast<const char*>(app.v) + roff, app.f32 != 0, lane);
      // the token's stores complete before this wave reads the tile back (waves of a
      // workgroup share the compute unit's L1, which the stores keep current)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    first_tile_keys();
  }

  const int vshift = (row * kStepTokens * BV) & 31;  // 0, or 16 for odd widths

  // Online softmax state per head: m = running maximum (base-2 log units, uniform
  // across the wave), l = per-lane partial sums of p (reduced once at the end).
  float m[G], l[G];
  float2 acc[G][PPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int j = 0; j < PPL; ++j) acc[g][j] = make_float2(0.f, 0.f);
  }
  // matrix-core mode: rotated-domain sums (cosine and sine elements; lane = pair, result
  // register = head), query operands (lane l: head l & 3 of each group of four), and
  // the wave's LDS rows of softmax weights [HG][4][64] and radius levels [64][16]
  f32x4 ax[M::HG], ay[M::HG];
  float qr[MXK && M::QREG ? M::HG : 1][MXK && M::QREG ? D : 1];
  const float* q_row[M::HG];
  // the waves' value rows follow the score table, if any: softmax weights and radius
  // levels as fp16, the matrix instructions' operand type
  _Float16* w_ph = reinterpret_cast<_Float16*>(s_union + TABLE_BYTES + wave * M::WAVE_BYTES);
  _Float16* w_lev = w_ph + M::PS_HALVES;
  if constexpr (MX) {
#pragma unroll
    for (int hg = 0; hg < M::HG; ++hg) {
      ax[hg] = ay[hg] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int h = 4 * hg + (lane & 3);
      q_row[hg] = s_q + min(h, G - 1) * D;
      if constexpr (MXK && M::QREG) {
#pragma unroll
        for (int e = 0; e < D; e += 4) {
          const float4 v = *reinterpret_cast<const float4*>(q_row[hg] + e);
          const bool on = h < G;  // rows past the group's heads stay zero
          qr[hg][e] = on ? v.x : 0.f;
          qr[hg][e + 1] = on ? v.y : 0.f;
          qr[hg][e + 2] = on ? v.z : 0.f;
          qr[hg][e + 3] = on ? v.w : 0.f;
        }
      }
      // weight rows of heads past G are zero for the whole launch
      if constexpr (MXV) {
#pragma unroll
        for (int g = G; g < 4 * M::HG; ++g) w_ph[(g >> 2) * 4 * kTile + (g & 3) * kTile + lane] = (_Float16)0.f;
      }
    }
  }

  for (; tile < tile_end; tile += NW) {
    // No register double-buffering: several waves per SIMD cover each other's load
    // latency, and the value planes are only requested once the scores are done, which
    // keeps the register count low enough for that occupancy.
    bool present = true;
    int idx = tile;
    if (ptab) {
      const int page = ptab[tile];
      present = page >= 0 && page < a.pg.num_pages;
      idx = present ? page : 0;
    }
    const uint8_t* tp = base + idx * stride;
    if (tile != tile_begin + wave) load_tile_keys<D, BK, BV>(cur, tp, lane);
    // opaque to the compiler, which otherwise specialises the whole tile body on an
    // absent tile and runs out of registers
    int nvalid = present ? min(seq_len - tile * kTile, kTile) : 0;
    asm volatile("" : "+s"(nvalid));
    const bool valid = lane < nvalid;

    // ---- keys: lane = token slot; sc[g] = the score of head g before the key scale
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    if constexpr (MXK) {
      // matrix cores: two chains, the cosine and the sine elements of each pair
      f32x4 sx[M::HG], sy[M::HG];
#pragma unroll
      for (int hg = 0; hg < M::HG; ++hg) sx[hg] = sy[hg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const uint32_t c = field<BK>(cur.ka, i);
        const float2 cs = lut_k[c];
        const float rho = (float)((cur.kr[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        const float bx = rho * cs.x, by = rho * cs.y;
#pragma unroll
        for (int hg = 0; hg < M::HG; ++hg) {
          float qa, qb;
          if constexpr (M::QREG) {
            qa = qr[hg][2 * i];
            qb = qr[hg][2 * i + 1];
          } else {
            const float2 qv = reinterpret_cast<const float2*>(q_row[hg])[i];
            qa = qv.x;
            qb = qv.y;
          }
          sx[hg] = mfma4x4(qa, bx, sx[hg]);
          sy[hg] = mfma4x4(qb, by, sy[hg]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g] = sx[g >> 2][g & 3] + sy[g >> 2][g & 3];
    } else if constexpr (TAB) {
      // Software pipeline over blocks of KB pairs: the table reads of block b + 1 are
      // issued before the FMAs of block b, so the LDS latency overlaps arithmetic
      // (the scheduling fences keep the compiler from re-serialising them).
      constexpr int KB = 4, NKB = P / KB;
      float tb[2][KB][G];
      uint32_t sg[2][KB];  // half table: sign bit of the radius (top code bit at bit 31)
#pragma unroll
      for (int blk = 0; blk <= NKB; ++blk) {
        if (blk < NKB) {
#pragma unroll
          for (int ii = 0; ii < KB; ++ii) {
            const int i = blk * KB + ii;
            const uint32_t c = field<BK>(cur.ka, i);
            sg[blk & 1][ii] = HALF ? (c >> (BK - 1)) << 31 : 0u;
            load_row<G>(tb[blk & 1][ii], ktab + (i * NTAB + (c & (NTAB - 1))) * G);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (blk > 0) {
#pragma unroll
          for (int ii = 0; ii < KB; ++ii) {
            const int i = (blk - 1) * KB + ii;
            float rho = (float)((cur.kr[i >> 2] >> (8 * (i & 3))) & 0xFFu);
            if (HALF) rho = __uint_as_float(__float_as_uint(rho) ^ sg[(blk - 1) & 1][ii]);
#pragma unroll
            for (int g = 0; g < G; ++g) sc[g] = fmaf(rho, tb[(blk - 1) & 1][ii][g], sc[g]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // q~ in chunks of CH pairs through scalar loads (2 * G * CH = 64 SGPRs); the
      // empty asm keeps the loads inside the tile loop
      constexpr int CH = 32 / G < P ? 32 / G : P;
#pragma unroll
      for (int i0 = 0; i0 < P; i0 += CH) {
        int qoff = 2 * i0;
        asm volatile("" : "+s"(qoff));
        const float* qc = qg + qoff;
#pragma unroll
        for (int ii = 0; ii < CH; ++ii) {
          const int i = i0 + ii;
          const uint32_t c = field<BK>(cur.ka, i);
          const float rho = (float)((cur.kr[i >> 2] >> (8 * (i & 3))) & 0xFFu);
          const float2 cs = lut_k[c];
          const float x = rho * cs.x, y = rho * cs.y;
#pragma unroll
          for (int g = 0; g < G; ++g)
            sc[g] = fmaf(x, qc[g * D + 2 * ii], fmaf(y, qc[g * D + 2 * ii + 1], sc[g]));
        }
      }
    }
    if constexpr (MXV)
      load_tile_values_mx(cur, tp, lane);
    else
      load_tile_values(cur, tp, lane, row, col);
    const float kscale = __half2float(__ushort_as_half((uint16_t)cur.ks));

    // ---- this lane's token's value radius: level(rho) = r0 2^(rho beta) with
    // r0 = s_min and beta = log2(s_max / s_min) / 15, or r0 = s_max and beta = 0 when
    // s_max <= s_min; r0 = 0 for slots past the end. Matrix-core values tabulate the 16
    // levels in the wave's LDS rows; the vector path folds r0 into the weights.
    float beta = 0.f, r0 = 0.f;
    {
      const float smin = __half2float(__ushort_as_half((uint16_t)(cur.vp & 0xFFFFu)));
      const float smax = __half2float(__ushort_as_half((uint16_t)(cur.vp >> 16)));
      r0 = smax;
      if (smax > smin) {
        r0 = smin;
        beta = (__log2f(smax) - __log2f(smin)) * (1.0f / 15.0f);
      }
      if (!valid) {
        r0 = 0.f;
        beta = 0.f;
      }
    }
    if constexpr (MXV) {
      // fp16 levels (in [2^-14, 65504] or 0), the operand type of the value products.
      // Up to four heads: four exponentials (levels 0, 4, 8, 12) and steps of 2^beta
      // between them, since the exponential is a quarter-rate instruction and three fp32
      // steps (a few ulp) vanish in the rounding to fp16 (1.5-2% per Mistral-7B-shaped
      // layer); at eight heads the extra live registers cost as much as that saves.
      h4x* dst = reinterpret_cast<h4x*>(w_lev + lane * 16);
      const float step = G <= 4 ? fast_exp2(beta) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        if constexpr (G <= 4) {
          const float l0 = r == 0 ? r0 : r0 * fast_exp2((float)r * beta);
          const float l1 = l0 * step, l2 = l1 * step, l3 = l2 * step;
          dst[r / 4] = h4x{(_Float16)l0, (_Float16)l1, (_Float16)l2, (_Float16)l3};
        } else {
          dst[r / 4] = h4x{(_Float16)(r0 * fast_exp2((float)r * beta)),
                           (_Float16)(r0 * fast_exp2((float)(r + 1) * beta)),
                           (_Float16)(r0 * fast_exp2((float)(r + 2) * beta)),
                           (_Float16)(r0 * fast_exp2((float)(r + 3) * beta))};
        }
      }
    }

    // ---- online softmax per head (lane = token), base 2; slots past the end get 0
    float pr[G];
    // new running maximum of head g from this tile's largest score; the sums so far are
    // rescaled to it (no token seen yet, only tiles of absent pages: nothing to rescale)
    auto raise_max = [&](int g, float tile_max) {
      const float mnew = fmaxf(m[g], tile_max);
      const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(m[g] - mnew);
      l[g] *= alpha;
      if constexpr (MXV) {
        ax[g >> 2][g & 3] *= alpha;
        ay[g >> 2][g & 3] *= alpha;
      } else {
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
          acc[g][j].x *= alpha;
          acc[g][j].y *= alpha;
        }
      }
      m[g] = mnew;
    };
    if constexpr (LAZY) {
      // Lazy maximum: the tile's weights are taken relative to the m of the tiles
      // before unless a score exceeds it by more than kLazyLog2 (a wave-wide vote); only
      // then are the wave maxima formed and the sums rescaled. Weights stay below
      // 2^kLazyLog2, inside the fp16 operand range, and the result, a ratio of sums
      // taken relative to the same m, does not depend on m.
      float s[G];
      bool up = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s[g] = valid ? sc[g] * kscale : -INFINITY;
        up = up || s[g] > m[g] + kLazyLog2;
      }
      if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) raise_max(g, wave_max(s[g]));
      }
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g] = s[g];
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        sc[g] = valid ? sc[g] * kscale : -INFINITY;
        raise_max(g, wave_max(sc[g]));
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pv = m[g] == -INFINITY ? 0.f : fast_exp2(sc[g] - m[g]);
      l[g] += pv;
      pr[g] = pv * r0;
      if constexpr (MXV) w_ph[(g >> 2) * 4 * kTile + (g & 3) * kTile + lane] = (_Float16)pv;
    }

    if constexpr (MXV) {
      // The wave's own LDS rows are read back by other lanes of the wave: LDS operations
      // of a wave complete in order, so only the compiler must keep them in order.
      asm volatile("" ::: "memory");
      // ---- values on the matrix cores: lane = pair (and token half for d = 64); one
      // product per token of the lane's half, weights of four tokens per LDS read
      const int th = D == 128 ? 0 : lane >> 5;
#pragma unroll
      for (int t4 = 0; t4 < M::VT / 4; ++t4) {
        h4x pa[M::HG];
#pragma unroll
        for (int hg = 0; hg < M::HG; ++hg)
          pa[hg] = *reinterpret_cast<const h4x*>(
              w_ph + hg * 4 * kTile + (lane & 3) * kTile + th * 32 + 4 * t4);
        // the four tokens' rebuilt elements level * (cos, sin), one packed fp16 product
        // each; four tokens per matrix instruction, fp32 sums
        h2x v2[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = 4 * t4 + u;
          const h2x cs = reinterpret_cast<const h2x*>(lut_v)[field<BV>(cur.va, t)];
          // up to four heads, one bit-field extract: the compiler would otherwise shift
          // and mask the pre-scaled nibble and add the row base separately (three
          // instructions; 2.4% per Mistral-7B-shaped layer). At eight heads the opaque
          // extract costs the schedule more than that (5-6% on the 70B-shaped layers).
          uint32_t rho;
          if constexpr (G <= 4)
            asm("v_bfe_u32 %0, %1, %2, 4" : "=v"(rho) : "v"(cur.vr[t >> 3]), "i"(4 * (t & 7)));
          else
            rho = (cur.vr[t >> 3] >> (4 * (t & 7))) & 0xFu;
          const _Float16 lvl = w_lev[(th * 32 + t) * 16 + rho];
          v2[u] = h2x{lvl, lvl} * cs;
        }
        const h4x bx = h4x{v2[0].x, v2[1].x, v2[2].x, v2[3].x};
        const h4x by = h4x{v2[0].y, v2[1].y, v2[2].y, v2[3].y};
#pragma unroll
        for (int hg = 0; hg < M::HG; ++hg) {
          ax[hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(pa[hg], bx, ax[hg], 0, 0, 0);
          ay[hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(pa[hg], by, ay[hg], 0, 0, 0);
        }
      }
      asm volatile("" ::: "memory");  // the next tile's LDS writes stay after these reads
    } else {
      // ---- values: lane (row, col); step k handles token slot 16 row + k
      uint32_t va[PPL][C::VAW];
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
#pragma unroll
        for (int w = 0; w < C::VAW; ++w) {
          if (BV & 1)
            va[j][w] = w + 1 < C::VAW ? __builtin_amdgcn_alignbit(cur.va[j][w + 1], cur.va[j][w], vshift)
                                      : (cur.va[j][w] >> vshift);
          else
            va[j][w] = cur.va[j][w];
        }
      }
      // Radius levels: at step k the 16 lanes of a row compute the 16 possible radii
      // 2^(level * beta) of their token (lane col takes level col), and each lane gathers
      // the levels of its pairs with a lane permute. The gather addresses are bytes
      // 4 * (16 row + level): low nibbles (even slots) and high nibbles (odd slots).
      uint32_t alo[PPL][2], ahi[PPL][2];
      const uint32_t rowb = 0x01010101u * (uint32_t)(64 * row);
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          alo[j][w] = ((cur.vr[j][w] & 0x0F0F0F0Fu) << 2) | rowb;
          ahi[j][w] = ((cur.vr[j][w] >> 2) & 0x3C3C3C3Cu) | rowb;
        }
      }
      const float colf = (float)col;
#pragma unroll
      for (int k = 0; k < kStepTokens; ++k) {
        // token slot 16 row + k: its softmax weights and radius step broadcast along the
        // row with DPP; the lane's level gathered from the row's 16 computed levels
        float pj[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pj[g] = row_bcast(pr[g], k);
        const float lev = fast_exp2(colf * row_bcast(beta, k));
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
          const float2 cs = lut_v[field<BV>(va[j], k)];
          const uint32_t aw = (k & 1) ? ahi[j][k >> 3] : alo[j][k >> 3];
          // the permute reads only address bits 2..7, so the byte needs no masking
          const float r = bperm_f((int)(aw >> (8 * ((k >> 1) & 3))), lev);
          const float vx = r * cs.x, vy = r * cs.y;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            acc[g][j].x = fmaf(pj[g], vx, acc[g][j].x);
            acc[g][j].y = fmaf(pj[g], vy, acc[g][j].y);
          }
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = wave_sum(l[g]);

  if constexpr (MXV) {
    // d = 64: the two token halves hold partial sums of the same pairs
    if constexpr (D == 64) {
#pragma unroll
      for (int hg = 0; hg < M::HG; ++hg)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ax[hg][r] += __shfl_xor(ax[hg][r], 32);
          ay[hg][r] += __shfl_xor(ay[hg][r], 32);
        }
    }
  } else {
    // ---- rows hold partial sums for the same pairs: fold them into row 0
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        acc[g][j].x += __shfl_xor(acc[g][j].x, 16);
        acc[g][j].y += __shfl_xor(acc[g][j].y, 16);
        acc[g][j].x += __shfl_xor(acc[g][j].x, 32);
        acc[g][j].y += __shfl_xor(acc[g][j].y, 32);
      }
    }
  }
  __syncthreads();  // every wave is done with the key table; reuse it for merging
  float* s_ml = reinterpret_cast<float*>(s_union);         // [NW][G][2]
  float* s_acc = s_ml + NW * G * 2;                          // [NW][G][D]
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_ml[(wave * G + g) * 2] = m[g];
      s_ml[(wave * G + g) * 2 + 1] = l[g];
    }
  }
  if constexpr (MXV) {
    if (lane < P) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        *reinterpret_cast<float2*>(s_acc + (wave * G + g) * D + 2 * lane) =
            make_float2(ax[g >> 2][g & 3], ay[g >> 2][g & 3]);
    }
  } else if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        const int e = 2 * (col * PPL + j);
        *reinterpret_cast<float2*>(s_acc + (wave * G + g) * D + e) = acc[g][j];
      }
    }
  }
  __syncthreads();
  const bool single = nsplit == 1;
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int g = idx / D, e = idx % D;
    float mm = s_ml[g * 2];
#pragma unroll
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, s_ml[(w * G + g) * 2]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = mm == -INFINITY ? 0.f : fast_exp2(s_ml[(w * G + g) * 2] - mm);
      ll += s_ml[(w * G + g) * 2 + 1] * f;
      aa += s_acc[(w * G + g) * D + e] * f;
    }
    if (single) {
      s_out[idx] = ll > 0.f ? aa / ll : 0.f;  // no token at all: zero output
    } else {
      // device-coherent stores (they bypass the non-coherent caches, so no cache
      // write-back is needed before another workgroup reads them)
      const size_t rowi = ((size_t)bk * G + g) * a.nsplit + split;
      __hip_atomic_store(a.part_acc + rowi * D + e, aa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (e == 0) {
        __hip_atomic_store(a.part_ml + 2 * rowi, mm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.part_ml + 2 * rowi + 1, ll, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (single) {
    __syncthreads();
    if (wave < G && lane < P) {
      const float2 v = reinterpret_cast<const float2*>(s_out)[wave * P + lane];
      store_output<D>(a, ((size_t)bk * G + wave) * D, lane, v.x, v.y);
    }
    return;
  }

  // ---- cross-split merge by the last workgroup of this (batch, kv head) to finish:
  // once its partial results are complete in memory it takes a ticket; the holder of
  // the last ticket combines the splits (log-sum-exp), applies the inverse transform
  // and resets the counter. The ordering rests on three properties of gfx950 rather
  // than on release/acquire fences (which here write back or invalidate the whole L2 of
  // an XCD and made the kernel 2-3x slower):
  //  1. the partials are stored and later loaded as agent-scope atomics, which the
  //     compiler emits with the device-coherence cache policy: they are performed past
  //     the per-XCD L2, so no stale copy of them can be read on another XCD;
  //  2. s_waitcnt vmcnt(0) returns only once those stores are acknowledged, i.e.
  //     performed at that coherence point, and it precedes the barrier after which one
  //     thread takes the ticket, so every store of the workgroup is performed first;
  //  3. the ticket is a system-scope atomic add, performed at memory in a single total
  //     order, so the workgroup that draws the last ticket does so after all others
  //     have performed their stores, and its coherent loads (1) then observe them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    // system scope: the counter update is performed at the memory side, so workgroups
    // on different XCDs (each with its own L2) count on one copy
    const unsigned t = __hip_atomic_fetch_add(a.tickets + bk, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_SYSTEM);
    *s_flag = t == (unsigned)(nsplit - 1);
  }
  __syncthreads();
  if (!*s_flag) return;
  // thread (g, e) folds element e of head g over the splits with a running
  // log-sum-exp. The partials come from other XCDs through memory, so every load of a
  // round is issued before any is used: 32 splits' worth at a time (a long single
  // sequence is cut into 32 splits or more) where the tile loop needs more registers
  // than that anyway (G >= 4), else 8, which keeps the small kernels' occupancy
  constexpr int MU = G >= 4 ? 32 : 8;
  auto ld = [](const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int g = idx / D, e = idx % D;
    const size_t row0 = ((size_t)bk * G + g) * a.nsplit;
    const float* ml = a.part_ml + 2 * row0;
    const float* pa = a.part_acc + row0 * D + e;
    float mm = -INFINITY, ll = 0.f, aa = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += MU) {
      float mv[MU], lv[MU], av[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int sp = min(s0 + u, nsplit - 1);
        mv[u] = ld(ml + 2 * sp);
        lv[u] = ld(ml + 2 * sp + 1);
        av[u] = ld(pa + (size_t)sp * D);
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
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
  __syncthreads();
  if (wave < G && lane < P) {
    const float2 v = reinterpret_cast<const float2*>(s_out)[wave * P + lane];
    store_output<D>(a, ((size_t)bk * G + wave) * D, lane, v.x, v.y);
  }
  if (tid == 0) __hip_atomic_store(a.tickets + bk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <int D, int G, int BK, int BV, int MODE>
hipError_t launch_mode(const AttnArgs& a, const AppendArgs& app, const uint8_t* cache, dim3 grid,
                       hipStream_t s) {
  if constexpr (attn_lds_bytes(D, G, BK, BV, MODE) <= kLdsBytesMax) {
    hipLaunchKernelGGL((attn_decode_kernel<D, G, BK, BV, MODE>), grid,
                       dim3(split_waves(MODE, G, D) * 64), 0, s, a, cache, a.qrot, app);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

// Launches the variant the host selected (a.key_table). Only the variants the host can
// select are compiled: those attn_mode gives for this code width (power-of-two n or
// not).
template <int D, int G, int BK, int BV>
hipError_t decode_launch(const AttnArgs& a, const AppendArgs& app, const uint8_t* cache, dim3 grid,
                    hipStream_t s) {
  constexpr int m_pow2 = attn_mode(D, G, 1 << BK, BK, BV);
  constexpr int m_other = attn_mode(D, G, (1 << BK) - 1, BK, BV);
  if (a.key_table == m_pow2) return launch_mode<D, G, BK, BV, m_pow2>(a, app, cache, grid, s);
  if constexpr (m_other != m_pow2) {
    if (a.key_table == m_other) return launch_mode<D, G, BK, BV, m_other>(a, app, cache, grid, s);
  }
#ifdef KVQ_ATTN_ALL_MODES
  switch (a.key_table) {
    case 0: return launch_mode<D, G, BK, BV, 0>(a, app, cache, grid, s);
    case 1: return launch_mode<D, G, BK, BV, 1>(a, app, cache, grid, s);
    case 2: return launch_mode<D, G, BK, BV, 2>(a, app, cache, grid, s);
    case 3: return launch_mode<D, G, BK, BV, 3>(a, app, cache, grid, s);
    case 5: return launch_mode<D, G, BK, BV, 5>(a, app, cache, grid, s);
    case 6: return launch_mode<D, G, BK, BV, 6>(a, app, cache, grid, s);
    case 7: return launch_mode<D, G, BK, BV, 7>(a, app, cache, grid, s);
    default: break;
  }
#endif
  return hipErrorInvalidValue;  // host and kernel disagree on the variant
}

template <int D, int G, int BK>
hipError_t decode_bv(const AttnArgs& a, const AppendArgs& app, const uint8_t* cache, dim3 grid,
                    hipStream_t s) {
  switch (a.bv) {
    case 6: return decode_launch<D, G, BK, 6>(a, app, cache, grid, s);
    case 7: return decode_launch<D, G, BK, 7>(a, app, cache, grid, s);
    case 8: return decode_launch<D, G, BK, 8>(a, app, cache, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int G>
hipError_t decode_bk(const AttnArgs& a, const AppendArgs& app, const uint8_t* cache, dim3 grid,
                    hipStream_t s) {
  switch (a.bk) {
    case 6: return decode_bv<D, G, 6>(a, app, cache, grid, s);
    case 7: return decode_bv<D, G, 7>(a, app, cache, grid, s);
    case 8: return decode_bv<D, G, 8>(a, app, cache, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t decode_g(const AttnArgs& a, const AppendArgs& app, const uint8_t* cache, dim3 grid,
                    hipStream_t s) {
  switch (a.group) {
    case 1: return decode_bk<D, 1>(a, app, cache, grid, s);
    case 2: return decode_bk<D, 2>(a, app, cache, grid, s);
    case 4: return decode_bk<D, 4>(a, app, cache, grid, s);
    case 8: return decode_bk<D, 8>(a, app, cache, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, const AppendArgs& app, int d,
                              const uint8_t* cache, hipStream_t stream) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  if ((a.key_table & 3) == 0) {  // scores read the rotated query from the workspace
    const dim3 pgrid((unsigned)(a.batch * a.hq));
    if (d == 64)
      hipLaunchKernelGGL(attn_prepare_kernel<64>, pgrid, dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_prepare_kernel<128>, pgrid, dim3(64), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.batch * a.hkv));
  return d == 64 ? decode_g<64>(a, app, cache, grid, stream)
                 : decode_g<128>(a, app, cache, grid, stream);
}

}  // namespace kvq
