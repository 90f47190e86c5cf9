"""bench.py's rocprofv3 summaries on synthetic CSVs (no GPU): kernel-name
normalisation, per-dispatch sums, the copy calibration and the HBM bytes per
launch written to traffic.json."""
import json

import bench


def test_kernel_short_name():
    assert bench.kernel_short_name(
        "void mxq::mxfp8_tile_kernel<true, true, true, 8, false>(mxq::Geometry, unsigned char*)"
    ) == "mxfp8_tile_kernel<true, true, true, 8, false>"
    assert bench.kernel_short_name("mxq::dequant_nvfp4_kernel(unsigned char const*, long)") == \
        "dequant_nvfp4_kernel"
    # a '(' inside template arguments is not the argument list
    assert bench.kernel_short_name("void k<f(int)>(int)") == "k<f(int)>"


def _csv(path, counter, rows):
    head = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
            '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
            '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
            '"Counter_Value","Start_Timestamp","End_Timestamp"')
    lines = [head]
    for disp, name, value in rows:
        lines.append(f'{disp},{disp},"Agent 1",1,1,1,64,1,"{name}",64,0,0,8,0,8,'
                     f'"{counter}",{value},0,1')
    path.write_text("\n".join(lines) + "\n")


def test_summarize_pmc(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda>(int)"
    kern = "mxq::dequant_nvfp4_kernel(unsigned char const*, long)"
    other = "void mxq::mxfp8_tile_kernel<true, true, false, 4, false>(mxq::Geometry)"
    # copy of 1 MiB: FETCH reads half the bytes in KiB (scale 2), WRITE all of them (scale 1)
    _csv(tmp_path / "f.csv", "FETCH_SIZE",
         [(1, copy, 512.0), (2, kern, 100.0), (2, kern, 20.0), (3, kern, 140.0), (4, other, 7.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE",
         [(1, copy, 1024.0), (2, kern, 300.0), (3, kern, 500.0), (4, other, 9.0)])
    run = {"legs": {"grouped_dequant_nvfp4": {"kernels": ["dequant_nvfp4_kernel"], "bytes": 555},
                    "act": {"kernels": ["mxfp8_tile_kernel<true, true, false, 4, false>"],
                            "bytes": 1},
                    "wgt": {"kernels": ["mxfp8_tile_kernel<true, true, false, 4, false>"],
                            "bytes": 2}},
           "copy_calibration": {"bytes": 2 << 20}}
    (tmp_path / "b.log").write_text("[bench] noise\n" + json.dumps(run) + "\n")
    out_j, out_t = tmp_path / "t.json", tmp_path / "t.txt"
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                        str(tmp_path / "b.log"), str(out_j), str(out_t))
    doc = json.loads(out_j.read_text())
    assert abs(doc["calibration"]["fetch_scale"] - 2.0) < 1e-12
    assert abs(doc["calibration"]["write_scale"] - 1.0) < 1e-12
    k = doc["kernels"]["dequant_nvfp4_kernel"]
    # dispatch 2 sums its two rows: fetch mean (120 + 140) / 2 = 130 KiB, write 400 KiB
    assert k["fetch_kib"] == 130.0 and k["write_kib"] == 400.0
    assert k["hbm_bytes_per_launch"] == 130 * 1024 * 2 + 400 * 1024
    assert k["leg"] == "grouped_dequant_nvfp4" and k["algorithmic_bytes"] == 555
    assert k["launches"] == 2
    assert k["source_digest"] == bench.kernel_digest("dequant_nvfp4_kernel")
    # a kernel shared by two legs of different sizes gets no entry
    assert "mxfp8_tile_kernel<true, true, false, 4, false>" not in doc["kernels"]
    assert "grouped_dequant_nvfp4" in out_t.read_text()


def test_summarize_stats(tmp_path):
    """Rows per (kernel, grid): one kernel launched on two shapes gives two
    rows; durations come from the trace's timestamps."""
    p = tmp_path / "t.csv"
    head = '"Kernel_Name","Grid_Size_X","Grid_Size_Y","Grid_Size_Z","Start_Timestamp","End_Timestamp"\n'
    rows = ['"void mxq::k<1>(int)",256,1,1,0,8000\n',
            '"void mxq::k<1>(int)",256,1,1,10000,18000\n',
            '"void mxq::k<1>(int)",1024,1,1,20000,22000\n',
            '"mxq::dequant_nvfp4_kernel(unsigned char const*)",64,1,1,30000,31000\n']
    p.write_text(head + "".join(rows))
    out = tmp_path / "s.txt"
    bench.summarize_stats(str(p), str(out), "title")
    lines = out.read_text().splitlines()
    body = [ln.split() for ln in lines if ln.startswith(("k<1>", "dequant_nvfp4_kernel"))]
    assert [b[0] for b in body] == ["k<1>", "k<1>", "dequant_nvfp4_kernel"]
    assert body[0][1:5] == ["256", "2", "8.00", "8.00"] and body[0][-1] == "84.2%"
    assert body[1][1:4] == ["1024", "1", "2.00"]
    assert body[2][1:4] == ["64", "1", "1.00"]



def test_code_text_drops_comments_only():
    """The traffic digests hash code_text: comments and whitespace runs go,
    string and character literals (which may hold comment markers) stay, and
    any change to the code itself changes the text."""
    src = ('int a = 1; // note\n/* block\n comment */ const char *s = "x//y /* z */";\n'
           "char q = '\"'; const char *e = \"\\\"//\";\n")
    assert bench.code_text(src) == ('int a = 1; const char *s = "x//y /* z */"; '
                                    "char q = '\"'; const char *e = \"\\\"//\";")
    assert bench.code_text(src) == bench.code_text(src.replace("note", "other words"))
    assert bench.code_text(src) != bench.code_text(src.replace("a = 1", "a = 2"))
    assert bench.code_text("x /* open") == "x"
