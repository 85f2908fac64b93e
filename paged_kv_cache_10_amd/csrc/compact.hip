// Conversion of exact pages into compact E4M3 pages and the CRC-32 of a
// compact page (the representation and layouts are described in compact.h).
//
// convert_kernel: one 256-thread work-group per (K|V x kv head, layer, page
// pair).  The exact block (32 KiB) is read once, in 1 KiB loads, into LDS
// while its largest magnitude is reduced; the 1,024 compact pieces are then
// built from LDS, each thread building whole 16-byte pieces from two exact
// pieces.
//
// crc_kernel: one 256-thread work-group per page.  In every layer thread t
// takes the t-th of 256 equal segments of the code region and computes its
// CRC from a zero register (table-driven, four bytes per step), reading its
// segment a 128-byte line at a time (the line's eight loads in flight
// together, so every line is fetched once); the 256
// segment CRCs are combined pairwise in a tree, using
//   crc(A || B) = crc(A) * x^(8|B|) + crc(B)   (mod the CRC polynomial),
// then the layer's scales are appended and the layers folded in order; the
// initial register 0xFFFFFFFF enters as its own advance over the page and
// the final xor is applied last.  This is the ordinary CRC-32 of the page's
// bytes: for each layer, its code blocks and then its scales.
#include "compact.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr uint32_t kCrcPoly = 0xEDB88320u;   // x^32 + ... (0x04C11DB7), bit-reversed

// E4M3 code of an FP32 value: nearest, ties to even, saturating at 448, the
// sign bit of the input kept.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (!(a < 464.f)) {
    code = 0x7Eu;                                   // at or past the rounding edge of 448
  } else if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.f);    // exact scaling, rint = half to even
  } else {
    const uint32_t ab = __float_as_uint(a);
    // keep 3 of 23 fraction bits, rounding half to even; a carry moves into
    // the exponent, which is what the next binade's code needs
    const uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;
    code = min(r - (120u << 3), 0x7Eu);             // exponent bias 127 -> 7
  }
  return sign | code;
}

__device__ __forceinline__ float bf16_elem(const uint4& u, int e) {
  const uint32_t w = (e < 2) ? u.x : (e < 4) ? u.y : (e < 6) ? u.z : u.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// Eight codes of x / s, packed little endian into two words.
__device__ __forceinline__ uint2 encode8(const uint4& u, float s) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e >> 2] |= e4m3_code(bf16_elem(u, e) / s) << (8 * (e & 3));
  return make_uint2(w[0], w[1]);
}

__global__ __launch_bounds__(256) void convert_kernel(ConvertArgs a) {
  const int kvh = blockIdx.x;              // 0 .. 2*Hkv-1: K heads, then V heads
  const int layer = blockIdx.y;
  const int i = blockIdx.z;
  const int tid = threadIdx.x;
  const int sp = a.src_pages[i];
  const int dp = a.dst_pages[i];
  if (sp < 0 || sp >= a.src_num_pages || dp < 0 || dp >= a.dst_num_pages) return;   // uniform

  const uint4* blk = reinterpret_cast<const uint4*>(
      a.src + ((int64_t)layer * a.src_num_pages + sp) * a.src_page_elems +
      (int64_t)kvh * kPageTokens * kHeadDim);
  uint8_t* out = a.codes + ((int64_t)layer * a.dst_num_pages + dp) * a.dst_page_bytes +
                 (int64_t)kvh * kCompactBlockBytes;

  // the block into LDS (piece p at p), reducing its largest magnitude
  __shared__ uint4 blk_lds[kPageTokens * kHeadDim / 8];
  float amax = 0.f;
#pragma unroll
  for (int m = 0; m < kPageTokens * kHeadDim / 8 / 256; ++m) {
    const uint4 u = load_stream(blk + tid + 256 * m);
    blk_lds[tid + 256 * m] = u;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf16_elem(u, e)));
  }
  amax = wave_max(amax);
  __shared__ float wmax[4];
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = (amax == 0.f) ? 1.f : amax / kE4M3Max;

  // 1,024 pieces of 16 codes
  const bool is_k = kvh < a.num_kv_heads;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int cp = tid + 256 * m;
    const int lane = cp & 63, q = lane >> 4;
    int p0, p1;
    if (is_k) {
      const int ld = cp >> 6, h = ld >> 3, t = (ld >> 2) & 1, kk = ld & 3, r = lane & 15;
      const int j = 32 * h + 8 * (r >> 2) + 4 * t + (r & 3);
      p0 = k_piece(j, 8 * kk + q);
      p1 = k_piece(j, 8 * kk + 4 + q);
    } else {
      const int d = 16 * (cp >> 6) + (lane & 15);
      p0 = v_piece(d, q);
      p1 = v_piece(d, 4 + q);
    }
    const uint2 lo = encode8(blk_lds[p0], s);
    const uint2 hi = encode8(blk_lds[p1], s);
    reinterpret_cast<uint4*>(out)[cp] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  if (tid == 0)
    a.scales[((int64_t)layer * a.dst_num_pages + dp) * 2 * a.num_kv_heads + kvh] = s;
}

// a * b modulo the CRC polynomial, both in the reflected representation
// (bit 31 is the coefficient of x^0).
__device__ __forceinline__ uint32_t gf_mul(uint32_t a, uint32_t b) {
  uint32_t p = 0;
  for (int i = 0; i < 32; ++i) {
    if (a & (0x80000000u >> i)) p ^= b;
    b = (b & 1u) ? (b >> 1) ^ kCrcPoly : (b >> 1);   // b *= x
  }
  return p;
}

__global__ __launch_bounds__(256) void crc_kernel(CrcArgs a) {
  __shared__ uint32_t tab[4][256];
  __shared__ uint32_t part[256];
  const int tid = threadIdx.x;
  // tab[0][v]: the register after one byte v from zero; tab[k]: k more zero bytes
  {
    uint32_t c = (uint32_t)tid;
    for (int b = 0; b < 8; ++b) c = (c & 1u) ? (c >> 1) ^ kCrcPoly : (c >> 1);
    tab[0][tid] = c;
  }
  __syncthreads();
  for (int k = 1; k < 4; ++k) {
    const uint32_t c = tab[k - 1][tid];
    tab[k][tid] = (c >> 8) ^ tab[0][c & 0xFFu];
    __syncthreads();
  }
  const int pg = a.pages[blockIdx.x];
  if (pg < 0 || pg >= a.num_pages) {                 // not a page of the pool: no CRC
    if (tid == 0) a.crc[blockIdx.x] = 0u;
    return;
  }
  const int64_t seg = a.page_bytes / 256;             // bytes per thread per layer
  uint32_t R = 0u;                                    // raw CRC of the layers so far
  for (int l = 0; l < a.num_layers; ++l) {
    const uint4* p = reinterpret_cast<const uint4*>(
        a.codes + ((int64_t)l * a.num_pages + pg) * a.page_bytes + (int64_t)tid * seg);
    uint32_t c = 0u;
    // ordinary loads: nontemporal ones would fetch the line again for each
    // of its eight 16-byte pieces (measured: 1.3x the bytes, twice the time)
    for (int64_t v0 = 0; v0 < seg / 16; v0 += 8) {     // one 128-byte line at a time
      uint4 line[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) line[v] = p[v0 + v];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const uint32_t w[4] = {line[v].x, line[v].y, line[v].z, line[v].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t x = c ^ w[k];
          c = tab[3][x & 0xFFu] ^ tab[2][(x >> 8) & 0xFFu] ^ tab[1][(x >> 16) & 0xFFu] ^
              tab[0][x >> 24];
        }
      }
    }
    part[tid] = c;
    __syncthreads();
    for (int k = 0; k < 8; ++k) {                      // pairs at distance 2^k
      const int d = 1 << k;
      uint32_t v = 0u;
      const bool left = (tid & (2 * d - 1)) == 0;
      if (left) v = gf_mul(part[tid], a.x_seg[k]) ^ part[tid + d];
      __syncthreads();
      if (left) part[tid] = v;
      __syncthreads();
    }
    if (tid == 0) {
      const uint8_t* sc = reinterpret_cast<const uint8_t*>(
          a.scales + ((int64_t)l * a.num_pages + pg) * a.scale_count);
      uint32_t d = 0u;
      for (int b = 0; b < 4 * a.scale_count; ++b) d = (d >> 8) ^ tab[0][(d ^ sc[b]) & 0xFFu];
      const uint32_t layer_raw = gf_mul(part[0], a.x_scales) ^ d;
      R = gf_mul(R, a.x_layer) ^ layer_raw;
    }
    __syncthreads();
  }
  if (tid == 0) a.crc[blockIdx.x] = R ^ a.init_term ^ 0xFFFFFFFFu;
}

}  // namespace

hipError_t launch_convert(const ConvertArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid(2 * a.num_kv_heads, a.num_layers, a.n);
  hipLaunchKernelGGL(convert_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_crc(const CrcArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(crc_kernel, dim3(a.n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
