// Direct global -> LDS tile loads (buffer_load ... lds) for gfx950 kernels.
#pragma once

#include "common.h"

namespace spr {

typedef int v4i32_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over one head's rows (byte offsets at or past `bytes`
// read as 0): base address, stride 0, num_records = bytes, raw dword format.
SPR_DEV v4i32_t head_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i32_t r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(int(bytes));
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from buffer offset `voff` straight into LDS at
// lds_addr + 16 * lane.  Issued in asm so the compiler's wait insertion does
// not pair it with later LDS reads of the other stage; completion is awaited
// explicitly (vmcnt) before the barrier that publishes the stage.  M0 (the
// LDS base) is declared clobbered, so the compiler restores it where it needs it.
SPR_DEV void lds_dma16(const v4i32_t& rsrc_in, uint32_t lds_addr, uint32_t voff) {
  // the descriptor must sit in SGPRs (it is wave-uniform by construction)
  v4i32_t rsrc;
  rsrc[0] = __builtin_amdgcn_readfirstlane(rsrc_in[0]);
  rsrc[1] = __builtin_amdgcn_readfirstlane(rsrc_in[1]);
  rsrc[2] = __builtin_amdgcn_readfirstlane(rsrc_in[2]);
  rsrc[3] = __builtin_amdgcn_readfirstlane(rsrc_in[3]);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// As lds_dma16, with a wave-uniform byte offset `soff` (SGPR) added to the
// per-lane offset: a load whose rows share one scalar base needs no per-lane
// address arithmetic.
SPR_DEV void lds_dma16_s(const v4i32_t& rsrc_in, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  v4i32_t rsrc;
  rsrc[0] = __builtin_amdgcn_readfirstlane(rsrc_in[0]);
  rsrc[1] = __builtin_amdgcn_readfirstlane(rsrc_in[1]);
  rsrc[2] = __builtin_amdgcn_readfirstlane(rsrc_in[2]);
  rsrc[3] = __builtin_amdgcn_readfirstlane(rsrc_in[3]);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(so)
      : "memory", "m0");
}

SPR_DEV uint32_t lds_addr_of(const void* p) {
  return uint32_t(reinterpret_cast<size_t>(
      (const __attribute__((address_space(3))) void*)(p)));
}

}  // namespace spr
