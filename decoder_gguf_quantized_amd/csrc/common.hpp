// Device helpers shared by the gfx950 kernels: wave64 reductions over DPP,
// fp16 scale loads, the argmax ordering and the Philox4x64-10 generator.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define QD_DEV __device__ __forceinline__

namespace qd {

constexpr int kWave = 64;

// Accumulator of a 32 x 32 MFMA tile (16 floats per lane).
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ggml type ids.  K-quant tensors are repacked at load into the 32-value block
// layouts of the legacy types; their scales stay in the file's precision:
//   Q4_K: Q4_0's nibble layout per 32-value sub-block; per sub-block a u16
//         (6-bit scale sc | 6-bit min m << 8) and per 256-value super-block a
//         u32 (fp16 d | fp16 dmin << 16); w = (d sc) n - (dmin m);
//   Q6_K: Q8_0's int8 layout (q - 32); per 16 values an int8 scale and per
//         super-block a u32 holding fp16 d; w = (d scale) q.
// The products d sc, dmin m, d scale are exact in f32.
constexpr int kF32 = 0;
constexpr int kQ4_0 = 2;
constexpr int kQ8_0 = 8;
constexpr int kQ4_K = 12;
constexpr int kQ6_K = 14;

// Where a layer's K/V row lives.  Contiguous (table null): [seq][nkv][ctx]
// rows.  Paged: [page][nkv][P] rows, P = 2^log2p positions per page, and
// sequence s's position j in page table[s * tw + j / P] (pages are handed out
// by the host; entries past a sequence's length hold any valid page).
struct KvMap {
  const int* table;     // paged: [seq][tw] page of each block of 2^log2p positions, else null
  int tw, log2p;
  int ring;             // contiguous sliding-window layer: log2 of its ring of positions
                        // (position j in slot j mod 2^ring), 0 = every position kept
};

// Row index (in head_dim units) of position j of KV head g of sequence s.
QD_DEV size_t kv_row(const KvMap& mp, int nkv, int ctx, int s, int g, int j) {
  if (mp.table) {
    const int pg = mp.table[s * mp.tw + (j >> mp.log2p)];
    return (((size_t)pg * nkv + g) << mp.log2p) + (j & ((1 << mp.log2p) - 1));
  }
  if (mp.ring) return (((size_t)s * nkv + g) << mp.ring) + (j & ((1 << mp.ring) - 1));
  return ((size_t)s * nkv + g) * ctx + j;
}

// Accumulator blocks per layer parity of decode attention's merge (chunk c adds
// into block c % kAccCopies; the O projection's input staging sums them).
constexpr int kAccCopies = 2;

// Types stored as 16 nibble bytes per 32-value block / as int8 per value.
constexpr bool nibble_layout(int qt) { return qt == kQ4_0 || qt == kQ4_K; }
constexpr bool int8_layout(int qt) { return qt == kQ8_0 || qt == kQ6_K; }

template <int CTRL, int ROW_MASK = 0xf>
QD_DEV float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}

// Sum over lane groups of G consecutive lanes (G in {8, 16, 32, 64}); every
// lane of a group receives its group's sum.
template <int G>
QD_DEV float group_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror: 8-lane sums
  if constexpr (G >= 16) v = dpp_add<0x140>(v);  // row_mirror: 16-lane sums
  if constexpr (G >= 32) v += __shfl_xor(v, 16);
  if constexpr (G >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Sum (MAX: maximum) of v over the lanes of the wave that hold the same place
// in groups of LG consecutive lanes (LG in {8, 16, 32}): lanes l, l + LG,
// l + 2 LG, ...; every lane receives its result.  Lanes move between 16-lane
// rows with gfx950's row swaps (v_permlane16_swap: odd rows of one operand
// with even rows of the other; v_permlane32_swap: the wave's halves), both
// plain VALU instructions, and within a row (LG = 8) with a DPP rotation.
template <bool MAX>
QD_DEV float lane_combine(float a, float b) { return MAX ? fmaxf(a, b) : a + b; }

template <int LG, bool MAX>
QD_DEV float stream_reduce(float v) {
  static_assert(LG == 8 || LG == 16 || LG == 32, "stream_reduce: LG in {8, 16, 32}");
  if constexpr (LG == 8) {  // lanes l and l ^ 8 of each row: rotate the row by 8
    const float r = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
    v = lane_combine<MAX>(v, r);
  }
  if constexpr (LG <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = lane_combine<MAX>(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return lane_combine<MAX>(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Full-wave sum, returned uniformly to every lane.
QD_DEV float wave_sum(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  v = dpp_add<0x140>(v);
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Two full-wave sums at once: every even lane receives the sum of a0 over the
// 64 lanes, every odd lane that of a1.  One exchange between lanes l and l ^ 1
// puts each value's pair sums into one register (even lanes a0's, odd lanes
// a1's), so the rest of the tree runs once: lanes l ^ 2, the quads of a row
// (rotations by 4 and 8, which keep the parity), then the rows (gfx950's row
// swaps, plain VALU instructions).
QD_DEV float pair_wave_sum(float a0, float a1, int lane) {
  const bool odd = lane & 1;
  const float keep = odd ? a1 : a0, send = odd ? a0 : a1;
  float t = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0xB1, 0xf, 0xf, true));
  t = dpp_add<0x4E>(t);   // quad_perm [2,3,0,1]: lanes l ^ 2
  t = dpp_add<0x124>(t);  // row_ror:4: the neighbouring quad
  t = dpp_add<0x128>(t);  // row_ror:8: the other two quads
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  t = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

QD_DEV float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

QD_DEV float half_bits_to_float(uint16_t h) {
  _Float16 f = __builtin_bit_cast(_Float16, h);
  return (float)f;
}

QD_DEV float load_half(const uint16_t* p) { return half_bits_to_float(*p); }

// Non-temporal loads for data read once per step (decode weights, KV cache):
// the streaming hint keeps them from displacing reused lines and sustains
// about 7.1 TB/s of plain reads on MI355X against about 6.3 TB/s for ordinary
// loads of the same pattern.
typedef uint32_t qd_u32x4 __attribute__((ext_vector_type(4)));
typedef float qd_f32x4 __attribute__((ext_vector_type(4)));
QD_DEV uint4 load_nt(const uint4* p) {
  const qd_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const qd_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
QD_DEV float4 load_nt(const float4* p) {
  const qd_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const qd_f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
QD_DEV float load_half_nt(const uint16_t* p) { return half_bits_to_float(__builtin_nontemporal_load(p)); }
QD_DEV float load_nt(const float* p) { return __builtin_nontemporal_load(p); }
QD_DEV uint32_t load_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
QD_DEV uint32_t load_nt(const uint16_t* p) { return __builtin_nontemporal_load(p); }
QD_DEV uint32_t load_nt(const int8_t* p) { return (uint32_t)(int32_t)__builtin_nontemporal_load(p); }

// K-quant scale pairs from their packed words: Q4_K (scale, min) of a
// sub-block from sm = sc | m << 8 and sd = d | dmin << 16; Q6_K scale from an
// int8 (sign-extended in sc) and sd = d.
QD_DEV float q4k_scale(uint32_t sm, uint32_t sd) { return half_bits_to_float((uint16_t)sd) * (float)(sm & 0xffu); }
QD_DEV float q4k_min(uint32_t sm, uint32_t sd) {
  return half_bits_to_float((uint16_t)(sd >> 16)) * (float)((sm >> 8) & 0xffu);
}
QD_DEV float q6k_scale(uint32_t sc, uint32_t sd) { return half_bits_to_float((uint16_t)sd) * (float)(int32_t)sc; }
typedef float qd_f32x2 __attribute__((ext_vector_type(2)));
QD_DEV float2 load_nt(const float2* p) {
  const qd_f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const qd_f32x2*>(p));
  return make_float2(v.x, v.y);
}

// v & m through an instruction the compiler cannot see into, so that it uses
// the masked word as written (whole-word masks whose bytes or fp16 halves are
// then read directly) instead of folding the mask into a bit-field extract per
// element.  Not volatile: the scheduler may move it like any other ALU op.
QD_DEV uint32_t opaque_and(uint32_t v, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(m));
  return r;
}

// Argmax ordering: (a, ia) ranks before (b, ib).  NaN ranks above every number,
// equal values go to the lower index.
QD_DEV bool ranks_before(float a, int ia, float b, int ib) {
  bool an = a != a, bn = b != b;
  if (an || bn) return an && bn ? ia < ib : an;
  return a > b || (a == b && ia < ib);
}

// The best (value, index) of the wave in ranks_before's order, in every lane.
QD_DEV void argmax_pair_wave(float& v, int& i) {
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (ranks_before(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 64x64->128
// multiplies with the paper's multipliers, key bumped by its Weyl constants.
struct u64x4 {
  uint64_t v[4];
};

QD_DEV u64x4 philox4x64_10(u64x4 c, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t hi0 = __umul64hi(M0, c.v[0]), lo0 = M0 * c.v[0];
    uint64_t hi1 = __umul64hi(M1, c.v[2]), lo1 = M1 * c.v[2];
    u64x4 n;
    n.v[0] = hi1 ^ c.v[1] ^ k0;
    n.v[1] = lo1;
    n.v[2] = hi0 ^ c.v[3] ^ k1;
    n.v[3] = lo0;
    c = n;
  }
  return c;
}

// Uniform in (0, 1) from the top 23 bits: ((r >> 41) + 0.5) * 2^-23, computed as
// the exact integer 2*(r>>41)+1 < 2^24 times 2^-24 (exact in f32).
QD_DEV float philox_uniform(uint64_t r) {
  uint32_t k = (uint32_t)(r >> 41) * 2u + 1u;
  return (float)k * 5.9604644775390625e-08f;  // 2^-24
}

}  // namespace qd
