// Blob layout planning shared by the host packer and the device packer: both
// write the same bytes, so the directory records, block offsets and the
// slot -> column order come from one place.
#pragma once
#include <stdint.h>

#include <vector>

#include "format.h"

namespace bitsmoe {

// Validates the shape and the widths and fills one directory record per
// expert (cmax left at 0) and the blob's total size.  Status as the C ABI.
int pack_plan(int E, int dout, int r, const uint8_t* bits, std::vector<DirRec>& dirs,
              uint64_t& total);

// Slot -> column list of one expert: width groups 1,2,3,4,6,8,16 in turn,
// ascending column index inside a group, each group padded with -1 to a
// multiple of 32 slots.
std::vector<int> pack_slot_columns(const uint8_t* bits_e, int r);

// The slot arrays of the component table of every expert (E *
// ctab_stride(r) bytes, the blob's bytes from ctab_offset(E)): slot of
// component k, kNoSlot for a 0-bit component.  Everything else zero.
void pack_ctab_slots(int E, int r, const uint8_t* bits, uint8_t* dst);

}  // namespace bitsmoe
