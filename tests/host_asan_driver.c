/*
 * Host-side checks of libiq under AddressSanitizer (host code only; the GPU
 * code is built as usual). Every call below is one that the library's
 * host-side validation answers by itself -- a rejected argument, a no-op size,
 * a host-only helper -- so nothing is launched and no GPU is needed. Pointers
 * that would be device memory are fake addresses that are never dereferenced.
 * Exit status: the number of calls whose status differs from the expected one.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "iq.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static iq_cache_view view(int32_t head_dim, int32_t hkv, int32_t cap, uintptr_t base, int32_t rotation,
                          int32_t k_bits) {
  iq_cache_view v;
  memset(&v, 0, sizeof v);
  v.head_dim = head_dim;
  v.num_kv_heads = hkv;
  v.capacity = cap;
  v.k_codes = (uint8_t*)base;
  v.v_codes = (uint8_t*)(base + 0x1000);
  v.k_norms = (float*)(base + 0x2000);
  v.v_norms = (float*)(base + 0x3000);
  v.rot = (const float*)(base + 0x4000);
  v.rotation = rotation;
  v.k_bits = k_bits;
  return v;
}

int main(void) {
  void* p = (void*)0x20000;
  void* odd = (void*)0x20004;

  /* host helpers */
  float c[16], t[15];
  expect("codebook", iq_codebook(c, t), IQ_OK);
  expect("codebook null", iq_codebook(NULL, t), IQ_ERR_INVALID_ARG);
  expect("codebook 16", iq_codebook_levels(16, c, t), IQ_OK);
  expect("codebook 8", iq_codebook_levels(8, c, t), IQ_OK);
  expect("codebook 12", iq_codebook_levels(12, c, t), IQ_ERR_INVALID_ARG);
  for (int s = 1; s >= -6; --s) {
    const char* str = iq_status_string((iq_status)s);
    if (str == NULL || strlen(str) == 0) {
      printf("FAIL status string %d\n", s);
      ++failures;
    }
  }

  /* append */
  iq_cache_view v = view(128, 2, 128, 0x10000, IQ_ROT_WHT_SO4, 3);
  iq_cache_view v64 = view(64, 2, 128, 0x10000, IQ_ROT_WHT_SO4, 3);
  iq_cache_view vcap = view(128, 2, 100, 0x10000, IQ_ROT_WHT_SO4, 3);
  iq_cache_view vmis = view(128, 2, 128, 0x10008, IQ_ROT_WHT_SO4, 3);
  iq_cache_view vrot = view(128, 2, 128, 0x10000, 3, 3);
  iq_cache_view vk5 = view(128, 2, 128, 0x10000, IQ_ROT_WHT_SO4, 5);
  expect("append null view", iq_rotate_quantize_append(NULL, p, p, IQ_F16, 4, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append d=64", iq_rotate_quantize_append(&v64, p, p, IQ_F16, 4, 0, NULL, NULL), IQ_ERR_UNSUPPORTED);
  expect("append dtype", iq_rotate_quantize_append(&v, p, p, (iq_dtype)7, 4, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append n<0", iq_rotate_quantize_append(&v, p, p, IQ_F16, -1, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append past cap", iq_rotate_quantize_append(&v, p, p, IQ_F16, 4, 125, NULL, NULL), IQ_ERR_CAPACITY);
  expect("append cap%32", iq_rotate_quantize_append(&vcap, p, p, IQ_F16, 4, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append null k", iq_rotate_quantize_append(&v, NULL, p, IQ_F16, 4, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append misaligned k", iq_rotate_quantize_append(&v, odd, p, IQ_F16, 4, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append misaligned cache", iq_rotate_quantize_append(&vmis, p, p, IQ_F16, 4, 0, NULL, NULL),
         IQ_ERR_INVALID_ARG);
  expect("append rotation", iq_rotate_quantize_append(&vrot, p, p, IQ_F16, 4, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append k_bits", iq_rotate_quantize_append(&vk5, p, p, IQ_F16, 4, 0, NULL, NULL), IQ_ERR_INVALID_ARG);
  expect("append no-op", iq_rotate_quantize_append(&v, p, p, IQ_F16, 0, 0, NULL, NULL), IQ_OK);

  /* decode */
  const size_t need = iq_decode_workspace_bytes(1, 8, 2, 100);
  if (need == 0) {
    printf("FAIL workspace bytes\n");
    ++failures;
  }
  expect("decode Hq%Hkv", iq_decode_attention(&v, p, 7, p, p, 1, 100, 0.1f, p, p, need, NULL), IQ_ERR_INVALID_ARG);
  expect("decode group 3", iq_decode_attention(&v, p, 6, p, p, 1, 100, 0.1f, p, p, need, NULL), IQ_ERR_UNSUPPORTED);
  expect("decode group 32", iq_decode_attention(&v, p, 64, p, p, 1, 100, 0.1f, p, p, need, NULL), IQ_ERR_UNSUPPORTED);
  expect("decode workspace", iq_decode_attention(&v, p, 8, p, p, 1, 100, 0.1f, p, p, need - 1, NULL),
         IQ_ERR_WORKSPACE);
  expect("decode n<0", iq_decode_attention(&v, p, 8, p, p, -1, 100, 0.1f, p, p, need, NULL), IQ_ERR_INVALID_ARG);
  expect("decode n=0", iq_decode_attention(&v, p, 8, p, p, 0, 100, 0.1f, p, p, need, NULL), IQ_OK);
  expect("decode grid", iq_decode_attention(&v, p, 8, p, p, 65536, 100, 0.1f, p, p, (size_t)1 << 40, NULL),
         IQ_ERR_UNSUPPORTED);
  expect("workspace bytes invalid", (int)iq_decode_workspace_bytes(-1, 8, 2, 100), 0);

  /* fp16 decode */
  expect("f16 cap%32", iq_decode_attention_f16(p, p, 256, 128, 2, 100, p, 8, p, p, 1, 100, 0.1f, p, p, need, NULL),
         IQ_ERR_INVALID_ARG);
  expect("f16 stride", iq_decode_attention_f16(p, p, 12, 128, 2, 128, p, 8, p, p, 1, 100, 0.1f, p, p, need, NULL),
         IQ_ERR_INVALID_ARG);
  expect("f16 group 3", iq_decode_attention_f16(p, p, 256, 128, 2, 128, p, 6, p, p, 1, 100, 0.1f, p, p, need, NULL),
         IQ_ERR_UNSUPPORTED);
  expect("f16 workspace",
         iq_decode_attention_f16(p, p, 256, 128, 2, 128, p, 8, p, p, 1, 100, 0.1f, p, p, need - 1, NULL),
         IQ_ERR_WORKSPACE);
  expect("f16 misaligned",
         iq_decode_attention_f16(odd, p, 256, 128, 2, 128, p, 8, p, p, 1, 100, 0.1f, p, p, need, NULL),
         IQ_ERR_INVALID_ARG);
  expect("f16 n=0", iq_decode_attention_f16(p, p, 256, 128, 2, 128, p, 8, p, p, 0, 100, 0.1f, p, p, need, NULL),
         IQ_OK);

  /* decode step, with and without a workspace */
  expect("step dtype", iq_append_decode_attention(&v, p, p, (iq_dtype)5, p, 8, p, p, 1, 100, 0.1f, p, p, need, NULL),
         IQ_ERR_INVALID_ARG);
  expect("step group 3", iq_append_decode_attention(&v, p, p, IQ_F16, p, 6, p, p, 1, 100, 0.1f, p, p, need, NULL),
         IQ_ERR_UNSUPPORTED);
  expect("step workspace",
         iq_append_decode_attention(&v, p, p, IQ_F16, p, 8, p, p, 1, 100, 0.1f, p, p, need - 1, NULL),
         IQ_ERR_WORKSPACE);
  expect("step null k", iq_append_decode_attention(&v, NULL, p, IQ_F16, p, 8, p, p, 1, 100, 0.1f, p, p, need, NULL),
         IQ_ERR_INVALID_ARG);
  expect("step n=0", iq_append_decode_attention(&v, p, p, IQ_F16, p, 8, p, p, 0, 100, 0.1f, p, p, need, NULL), IQ_OK);
  iq_cache_view v4 = view(128, 4, 128, 0x10000, IQ_ROT_WHT_SO4, 3);
  if (iq_decode_workspace_bytes(64, 32, 4, 32768) <= IQ_NOALLOC_SCRATCH_BYTES) {
    printf("FAIL oversized records fit the scratch\n");
    ++failures;
  }
  expect("noalloc oversized", iq_append_decode_attention_noalloc(&v4, p, p, IQ_F16, p, 32, p, p, 64, 32768, 0.1f, p,
                                                                 NULL),
         IQ_ERR_WORKSPACE);
  expect("noalloc group 3", iq_append_decode_attention_noalloc(&v4, p, p, IQ_F16, p, 12, p, p, 1, 100, 0.1f, p, NULL),
         IQ_ERR_UNSUPPORTED);
  expect("noalloc null k", iq_append_decode_attention_noalloc(&v4, NULL, p, IQ_F16, p, 32, p, p, 1, 100, 0.1f, p, NULL),
         IQ_ERR_INVALID_ARG);
  expect("noalloc n=0", iq_append_decode_attention_noalloc(&v4, p, p, IQ_F16, p, 32, p, p, 0, 100, 0.1f, p, NULL),
         IQ_OK);

  /* deferred decode */
  const size_t dneed = iq_decode_deferred_workspace_bytes(1, 8, 2, 300, 100);
  expect("deferred workspace", iq_decode_attention_deferred(&v, p, p, 100, p, p, 256, 128, 320, p, p, 300, p, 8, 1,
                                                            0.1f, p, p, dneed - 1, NULL),
         IQ_ERR_WORKSPACE);
  expect("deferred cap16", iq_decode_attention_deferred(&v, p, p, 100, p, p, 256, 128, 300, p, p, 300, p, 8, 1, 0.1f,
                                                        p, p, dneed, NULL),
         IQ_ERR_INVALID_ARG);
  expect("deferred group 3", iq_decode_attention_deferred(&v, p, p, 100, p, p, 256, 128, 320, p, p, 300, p, 6, 1,
                                                          0.1f, p, p, dneed, NULL),
         IQ_ERR_UNSUPPORTED);
  expect("deferred n=0", iq_decode_attention_deferred(&v, p, p, 100, p, p, 256, 128, 320, p, p, 300, p, 8, 0, 0.1f, p,
                                                      p, dneed, NULL),
         IQ_OK);

  /* dequantize, rotate, quantize-pack */
  expect("dequant capacity", iq_dequantize(&v, 120, 20, IQ_F32, p, p, NULL), IQ_ERR_CAPACITY);
  expect("dequant dtype", iq_dequantize(&v, 0, 20, (iq_dtype)3, p, p, NULL), IQ_ERR_INVALID_ARG);
  expect("dequant no outputs", iq_dequantize(&v, 0, 20, IQ_F32, NULL, NULL, NULL), IQ_OK);
  expect("rotate null", iq_rotate(NULL, 0, 1, p, p, 4, 0, NULL), IQ_ERR_INVALID_ARG);
  expect("rotate inverse flag", iq_rotate(p, 0, 1, p, p, 4, 2, NULL), IQ_ERR_INVALID_ARG);
  expect("rotate kind", iq_rotate(p, 3, 1, p, p, 4, 0, NULL), IQ_ERR_INVALID_ARG);
  expect("rotate n=0", iq_rotate(p, 2, 1, p, p, 0, 0, NULL), IQ_OK);
  expect("quantize n<0", iq_quantize_pack(p, -1, p, p, NULL), IQ_ERR_INVALID_ARG);
  expect("quantize n=0", iq_quantize_pack(p, 0, p, p, NULL), IQ_OK);

  printf("%d failure(s)\n", failures);
  return failures;
}
