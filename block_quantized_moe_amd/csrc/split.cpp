// Host-side loader split: on-disk (array-of-structs) quant blocks -> the
// GPU-resident struct-of-arrays tensors the kernels read.
//
// The GGUF block-dequant page ("Design -- CPU-side decomposition") splits each
// on-disk block once at load time into separate GPU-resident tensors (packed
// codes, scales, lookup tables) so the hot kernels do no per-call byte
// surgery; the DSV4 campaign page repacks q2_K blocks to SoA at load because
// the AoS code bytes sit at 84*blk+16 and are only 4-byte aligned.  Here every
// output array is naturally aligned, and the matmul formats are tiled by
// 16-row blocks for coalesced wave-wide loads.  Any row count is accepted:
// the tiled arrays are sized for rows rounded up to a multiple of 16
// (qmoe_split_rows), and the rows past the end are written as zeros, so the
// kernels may read a whole 16-row block even where its tail holds no row.
#include <stdint.h>
#include <string.h>

#include "../../include/qmoe.h"

static inline int64_t pad16(int64_t rows) { return (rows + 15) / 16 * 16; }

extern "C" {

int64_t qmoe_split_rows(int64_t rows) { return rows < 0 ? -1 : pad16(rows); }

// Q8_0: codes tiled as [R/16][k/64][4][16][16] (chunk c of 16 values of row
// 16 rb + r in k tile kt), block scales as [R/16][k/32][16].
int qmoe_split_q8_0(const void* aos, int64_t rows, int64_t k, int8_t* qs, uint16_t* d) {
  if (!aos || !qs || !d || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (k % 64) return QMOE_ERR_BLOCK;
  const int64_t KT = k / 64, NB = k / 32;
  memset(qs + rows / 16 * 16 * k, 0, (size_t)((pad16(rows) - rows / 16 * 16) * k));
  memset(d + rows / 16 * 16 * NB, 0, (size_t)((pad16(rows) - rows / 16 * 16) * NB) * 2);
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t b = 0; b < NB; ++b) {
      const uint8_t* p = (const uint8_t*)aos + (R * NB + b) * 34;
      memcpy(&d[(rb * NB + b) * 16 + r], p, 2);
      for (int h = 0; h < 2; ++h) {  // the block's two 16-value chunks
        const int64_t kk = 32 * b + 16 * h, kt = kk / 64, c = (kk % 64) / 16;
        memcpy(&qs[(((rb * KT + kt) * 4 + c) * 16 + r) * 16], p + 2 + 16 * h, 16);
      }
    }
  }
  return QMOE_OK;
}

// FP8 block weights: E4M3 codes [rows][k], one byte per weight, tiled like
// the Q8_0 codes ([R/16][k/64][4][16][16]: chunk c of 16 values of row
// 16 rb + r in k tile kt).  The fp32 block scales [rows/128][k/128] are used
// as they are.
int qmoe_split_fp8(const uint8_t* w, int64_t rows, int64_t k, uint8_t* qs) {
  if (!w || !qs || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (rows % 128 || k % 128) return QMOE_ERR_BLOCK;
  const int64_t KT = k / 64;
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t kt = 0; kt < KT; ++kt)
      for (int c = 0; c < 4; ++c)
        memcpy(&qs[(((rb * KT + kt) * 4 + c) * 16 + r) * 16], w + R * k + 64 * kt + 16 * c, 16);
  }
  return QMOE_OK;
}

// MXFP4: 17-byte blocks (E8M0 exponent, 16 code bytes with element 2i in the
// low nibble of byte i).  Codes tiled as u32 [R/16][k/64][2][16][4]: word w
// of block j of row 16 rb + r holds elements 8w .. 8w+7 with element 8w+i in
// nibble i (code bytes 4w .. 4w+3 as they are on disk, so a per-byte
// conversion yields pairs in k order); exponents as [R/16][k/32][16].
int qmoe_split_mxfp4(const void* aos, int64_t rows, int64_t k, uint32_t* qs, uint8_t* e) {
  if (!aos || !qs || !e || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (k % 64) return QMOE_ERR_BLOCK;
  const int64_t KT = k / 64, NB = k / 32;
  memset(qs + rows / 16 * 16 * k / 8, 0, (size_t)((pad16(rows) - rows / 16 * 16) * k / 8) * 4);
  memset(e + rows / 16 * 16 * NB, 0, (size_t)((pad16(rows) - rows / 16 * 16) * NB));
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t b = 0; b < NB; ++b) {
      const uint8_t* p = (const uint8_t*)aos + (R * NB + b) * 17;
      e[(rb * NB + b) * 16 + r] = p[0];
      uint8_t code[32];
      for (int i = 0; i < 16; ++i) {
        code[2 * i] = p[1 + i] & 15;
        code[2 * i + 1] = p[1 + i] >> 4;
      }
      uint32_t* dst = qs + (((rb * KT + b / 2) * 2 + (b % 2)) * 16 + r) * 4;
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
        for (int i = 0; i < 4; ++i)
          word |= (uint32_t)(code[8 * w + 2 * i] | (code[8 * w + 2 * i + 1] << 4)) << (8 * i);
        dst[w] = word;
      }
    }
  }
  return QMOE_OK;
}

// Q2_K and IQ2_XXS are tiled by 16-row blocks (global row R = 16 rb + r),
// super-block sb = k / 256 inner, so that every 64-wide k tile of a 16-row
// block reads its codes and per-row metadata as a few contiguous runs (the
// layouts are spelled out in qmoe.h).  aos holds rows * k/256 blocks, row
// after row.
int qmoe_split_q2_k(const void* aos, int64_t rows, int64_t k, uint32_t* qs, uint8_t* scales,
                    uint16_t* d, uint16_t* dmin) {
  if (!aos || !qs || !scales || !d || !dmin || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  const int64_t SB = k / 256;
  uint8_t* qb = (uint8_t*)qs;
  {
    const int64_t r0 = rows / 16 * 16, np = pad16(rows) - r0;  // rows of the last, partial block
    memset(qb + r0 * SB * 64, 0, (size_t)(np * SB * 64));
    memset(scales + r0 * SB * 16, 0, (size_t)(np * SB * 16));
    memset(d + r0 * SB, 0, (size_t)(np * SB) * 2);
    memset(dmin + r0 * SB, 0, (size_t)(np * SB) * 2);
  }
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t sb = 0; sb < SB; ++sb) {
      const uint8_t* p = (const uint8_t*)aos + (R * SB + sb) * 84;
      const int64_t base = rb * SB + sb;
      memcpy(&scales[(base * 16 + r) * 16], p, 16);
      for (int h = 0; h < 2; ++h) memcpy(&qb[((base * 2 + h) * 16 + r) * 32], p + 16 + 32 * h, 32);
      memcpy(&d[base * 16 + r], p + 80, 2);
      memcpy(&dmin[base * 16 + r], p + 82, 2);
    }
  }
  return QMOE_OK;
}

// Q4_K (the pages name the format only; read as the GGUF k-quant block):
// 144-byte blocks [fp16 d][fp16 dmin][12 packed bytes of six-bit sub-block
// scales and mins][128 code bytes: element e in byte 32*(e/64) + e%32, low
// nibble when e%64 < 32].  Tiled, t = (R/16) * k/256 + super-block, r = R%16:
// qs [t][4][16][32] (quarter h of row r = its code bytes 32h .. 32h+31),
// scales [t][16][16] (row r's 8 scales, then its 8 mins, one byte each),
// d, dmin [t][16].
int qmoe_split_q4_k(const void* aos, int64_t rows, int64_t k, uint8_t* qs, uint8_t* scales, uint16_t* d,
                    uint16_t* dmin) {
  if (!aos || !qs || !scales || !d || !dmin || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  const int64_t SB = k / 256;
  {
    const int64_t r0 = rows / 16 * 16, np = pad16(rows) - r0;  // rows of the last, partial block
    memset(qs + r0 * SB * 128, 0, (size_t)(np * SB * 128));
    memset(scales + r0 * SB * 16, 0, (size_t)(np * SB * 16));
    memset(d + r0 * SB, 0, (size_t)(np * SB) * 2);
    memset(dmin + r0 * SB, 0, (size_t)(np * SB) * 2);
  }
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t sb = 0; sb < SB; ++sb) {
      const uint8_t* p = (const uint8_t*)aos + (R * SB + sb) * 144;
      const int64_t base = rb * SB + sb;
      memcpy(&d[base * 16 + r], p, 2);
      memcpy(&dmin[base * 16 + r], p + 2, 2);
      const uint8_t* b = p + 4;
      uint8_t* sm = &scales[(base * 16 + r) * 16];
      for (int j = 0; j < 4; ++j) {
        sm[j] = b[j] & 63;
        sm[8 + j] = b[j + 4] & 63;
        sm[j + 4] = (uint8_t)((b[j + 8] & 15) | ((b[j] >> 6) << 4));
        sm[8 + j + 4] = (uint8_t)((b[j + 8] >> 4) | ((b[j + 4] >> 6) << 4));
      }
      for (int h = 0; h < 4; ++h) memcpy(&qs[((base * 4 + h) * 16 + r) * 32], p + 16 + 32 * h, 32);
    }
  }
  return QMOE_OK;
}

// Q6_K (named only; read as the GGUF k-quant block): 210-byte blocks [128
// bytes of low nibbles][64 bytes of top bit pairs][16 int8 scales][fp16 d];
// element e = 128n + 32p + l takes its low 4 bits from byte 64n + 32(p%2) + l
// of the first array (high nibble when p >= 2) and its top 2 bits from byte
// 32n + l of the second (bits 2p, 2p+1).  Tiled: qs [t][4][16][32] low
// nibbles in the Q4_K code arrangement (byte i of quarter h: element 64h+i
// in the low nibble, 64h+32+i in the high), qh [t][2][16][32] top bit pairs
// as on disk (half n of row r = its bytes 32n .. 32n+31), scales int8
// [t][16][16], d [t][16].
int qmoe_split_q6_k(const void* aos, int64_t rows, int64_t k, uint8_t* qs, uint8_t* qh, int8_t* scales,
                    uint16_t* d) {
  if (!aos || !qs || !qh || !scales || !d || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  const int64_t SB = k / 256;
  {
    const int64_t r0 = rows / 16 * 16, np = pad16(rows) - r0;
    memset(qs + r0 * SB * 128, 0, (size_t)(np * SB * 128));
    memset(qh + r0 * SB * 64, 0, (size_t)(np * SB * 64));
    memset(scales + r0 * SB * 16, 0, (size_t)(np * SB * 16));
    memset(d + r0 * SB, 0, (size_t)(np * SB) * 2);
  }
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t sb = 0; sb < SB; ++sb) {
      const uint8_t* p = (const uint8_t*)aos + (R * SB + sb) * 210;
      const int64_t base = rb * SB + sb;
      uint8_t lo[256];
      for (int e = 0; e < 256; ++e) {
        const int n = e / 128, pp = (e % 128) / 32, l = e % 32;
        const uint8_t b = p[64 * n + 32 * (pp % 2) + l];
        lo[e] = pp < 2 ? (b & 15) : (b >> 4);
      }
      for (int h = 0; h < 4; ++h)
        for (int i = 0; i < 32; ++i)
          qs[((base * 4 + h) * 16 + r) * 32 + i] = (uint8_t)(lo[64 * h + i] | (lo[64 * h + 32 + i] << 4));
      for (int n = 0; n < 2; ++n) memcpy(&qh[((base * 2 + n) * 16 + r) * 32], p + 128 + 32 * n, 32);
      memcpy(&scales[(base * 16 + r) * 16], p + 192, 16);
      memcpy(&d[base * 16 + r], p + 208, 2);
    }
  }
  return QMOE_OK;
}

int qmoe_split_iq2_xxs(const void* aos, int64_t rows, int64_t k, uint32_t* ia, uint16_t* d) {
  if (!aos || !ia || !d || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  const int64_t SB = k / 256;
  {
    const int64_t r0 = rows / 16 * 16, np = pad16(rows) - r0;
    memset(ia + r0 * SB * 16, 0, (size_t)(np * SB * 16) * 4);
    memset(d + r0 * SB, 0, (size_t)(np * SB) * 2);
  }
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t sb = 0; sb < SB; ++sb) {
      const uint8_t* p = (const uint8_t*)aos + (R * SB + sb) * 66;
      const int64_t base = rb * SB + sb;
      memcpy(&d[base * 16 + r], p, 2);
      for (int g = 0; g < 8; ++g) {
        memcpy(&ia[((base * 8 + g) * 16 + r) * 2], p + 2 + 8 * g, 4);      // grid indices
        memcpy(&ia[((base * 8 + g) * 16 + r) * 2 + 1], p + 6 + 8 * g, 4);  // signs | scale
      }
    }
  }
  return QMOE_OK;
}

// Nibble order inside a word: element 2i -> nibble i, element 2i+1 -> nibble 4+i.
static uint32_t int4_gpu_word(uint32_t v) {
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    r |= ((v >> (8 * i)) & 0xFu) << (4 * i);
    r |= ((v >> (8 * i + 4)) & 0xFu) << (4 * i + 16);
  }
  return r;
}

int qmoe_split_int4(const uint32_t* words, const uint16_t* scales, const uint16_t* biases,
                    int64_t rows, int64_t k, int32_t group, uint32_t* qs_out, uint32_t* sb_out) {
  if (!words || !scales || !biases || !qs_out || !sb_out || rows < 0 || k < 0) return QMOE_ERR_ARG;
  if (!(group == 32 || group == 64 || group == 128 || group == 256)) return QMOE_ERR_BLOCK;
  if (k % 64 || k % group) return QMOE_ERR_BLOCK;
  const int64_t kt_n = k / 64, wpr = k / 8, G = k / group;
  {
    const int64_t r0 = rows / 16 * 16, np = pad16(rows) - r0;
    memset(qs_out + r0 * wpr, 0, (size_t)(np * wpr) * 4);
    memset(sb_out + r0 * G, 0, (size_t)(np * G) * 4);
  }
  for (int64_t R = 0; R < rows; ++R) {
    const int64_t rb = R / 16, r = R % 16;
    for (int64_t kt = 0; kt < kt_n; ++kt)
      for (int g = 0; g < 4; ++g)
        for (int w = 0; w < 2; ++w) {
          const int64_t src = R * wpr + kt * 8 + g * 2 + w;          // word of k = 64kt + 16g + 8w
          const int64_t dst = ((rb * kt_n + kt) * 64 + (16 * g + r)) * 2 + w;
          qs_out[dst] = int4_gpu_word(words[src]);
        }
    for (int64_t gi = 0; gi < G; ++gi)
      sb_out[(rb * G + gi) * 16 + r] = (uint32_t)scales[R * G + gi] | ((uint32_t)biases[R * G + gi] << 16);
  }
  return QMOE_OK;
}

void qmoe_iq2_signs_table(uint8_t out[128]) {
  if (!out) return;
  for (int i = 0; i < 128; ++i) {
    const int odd = __builtin_popcount((unsigned)i) & 1;
    out[i] = (uint8_t)(i | (odd << 7));
  }
}

}  // extern "C"
